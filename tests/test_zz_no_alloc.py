"""kie_prefill_batched_noalloc against kie_prefill_batched.

The no-allocation entry runs the same kernels with its workspace in the
library's static device array instead of the handle's; when the usual chunk
does not fit the array it takes smaller chunks, which changes no arithmetic
(each product's sums run over the same operands in the same order, and the
causal attention walks the cache from position 0 whatever the chunk).  So
the K/V rows it writes and the decode that follows must equal the
allocating entry's bit for bit: two calls in a row on the same handles, the
second with a shorter prompt.  The 2b widths need about 134 KiB of
workspace per position, so a 512-token prompt takes two chunks of the
64 MiB array; the MoE widths about 250 KiB, so its 300-token prompt does
too.  Calls go through the C ABI (the Engine binding only marshals).
"""
import sys

import numpy as np
import pytest

from kie_synth import get_config, make_prompt, make_weights

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    return t


@pytest.fixture(scope="module")
def kie():
    import persistent_decode_monokernel_amd as k
    k.load()
    return k


def _same_prefill_and_decode(torch, kie, a, b, cfg, prompt, n_decode=3):
    a.reset()
    b.reset()
    a.prefill_batched(prompt)
    b.prefill_batched_noalloc(prompt)
    assert a.position == b.position == len(prompt) - 1
    P = len(prompt) - 1
    for l in range(cfg.n_layers):
        ka, va = a.read_kv(l, 0, P)
        kb, vb = b.read_kv(l, 0, P)
        assert np.array_equal(ka.view(np.uint16), kb.view(np.uint16)), ("K", l)
        assert np.array_equal(va.view(np.uint16), vb.view(np.uint16)), ("V", l)
    ta, za = a.decode(n_decode, logits=True)
    tb, zb = b.decode(n_decode, logits=True)
    assert np.array_equal(ta.cpu().numpy(), tb.cpu().numpy())
    assert np.array_equal(za.cpu().numpy().view(np.uint32), zb.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("name,layers,lengths", [("2b", 3, (512, 130)), ("moe", 2, (300, 40))])
def test_noalloc_prefill_matches_the_allocating_entry(torch, kie, name, layers, lengths):
    cfg = get_config(name, n_layers=layers)
    _say("no-alloc prefill", name, layers, lengths)
    W = make_weights(cfg, seed=3, device="cuda")
    a = kie.Engine(cfg, W, max_seq=max(lengths) + 8)
    b = kie.Engine(cfg, W, max_seq=max(lengths) + 8)
    try:
        for n in lengths:            # two calls in a row, the second shorter
            prompt = make_prompt(cfg, seed=n, length=n)
            _same_prefill_and_decode(torch, kie, a, b, cfg, prompt)
    finally:
        a.close()
        b.close()
