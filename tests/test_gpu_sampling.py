"""GPU temperature sampling (kie_decode_sampled) against the oracle's sampler.

The kernel's draw is recomputed by oracle.sampling from the kernel's own
logits (same Philox words, same float64 key, same first-maximum rule); the
logits themselves are checked against a teacher-forced oracle replay.
"""
import sys

import numpy as np
import pytest

from kie_synth import get_config, make_prompt, make_weights, weights_to_numpy
from oracle import Oracle
from oracle.sampling import sample_keys, sample_token
from tests.parity import KEY_MARGIN, compare_sampled_steps

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


def _sampled(kie, cfg, W, prompt, n, seed, temperature, **kw):
    eng = kie.Engine(cfg, W, **kw)
    eng.prefill(prompt)
    toks, z = eng.decode(n, seed=seed, temperature=temperature)
    return eng, toks.cpu().numpy(), z.cpu().numpy()


@pytest.mark.parametrize("temperature,seed", [(0.8, 1234), (1.5, 2**63 + 17), (0.05, 7)])
def test_tiny_sampled_decode_matches_oracle_sampler(torch, kie, temperature, seed):
    cfg = get_config("tiny")
    _say("tiny sampled", temperature, seed)
    W = make_weights(cfg, seed=0, device="cuda")
    prompt = make_prompt(cfg)
    n = 24
    eng, toks, z = _sampled(kie, cfg, W, prompt, n, seed, temperature)
    P = len(prompt)
    assert eng.position == P - 1 + n
    o = Oracle(cfg, weights_to_numpy(W))
    o.prefill(prompt)
    _, zo = o.decode(n, force=toks)
    rep = compare_sampled_steps(z, toks, zo, temperature, seed, P - 1)
    _say(rep)
    assert rep["pinned"] >= n - 2
    eng.close()


def test_sampled_decode_is_deterministic_composable_and_seeded(torch, kie):
    cfg = get_config("tiny")
    _say("tiny sampled determinism")
    W = make_weights(cfg, seed=0, device="cuda")
    prompt = make_prompt(cfg)
    _, t1, z1 = _sampled(kie, cfg, W, prompt, 30, 99, 1.0)
    _, t2, z2 = _sampled(kie, cfg, W, prompt, 30, 99, 1.0)
    np.testing.assert_array_equal(t1, t2)
    np.testing.assert_array_equal(z1, z2)
    # decode(a) then decode(b) equals decode(a + b): the draw depends on the
    # seed and the position only
    eng = kie.Engine(cfg, W)
    eng.prefill(prompt)
    ta, _ = eng.decode(11, seed=99, temperature=1.0)
    tb, _ = eng.decode(19, seed=99, temperature=1.0)
    np.testing.assert_array_equal(np.concatenate([ta.cpu().numpy(), tb.cpu().numpy()]), t1)
    eng.close()
    # the staged (graph) mode runs the same lm_head stage: identical draws
    _, tg, zg = _sampled(kie, cfg, W, prompt, 30, 99, 1.0, graph=True)
    np.testing.assert_array_equal(tg, t1)
    np.testing.assert_array_equal(zg, z1)
    # another seed gives another sequence (tiny vocab 512 at T = 1: the
    # chance of 30 equal draws is negligible)
    _, t3, _ = _sampled(kie, cfg, W, prompt, 30, 100, 1.0)
    assert not np.array_equal(t3, t1)


def test_zero_temperature_is_greedy_and_bad_temperatures_are_rejected(torch, kie):
    cfg = get_config("tiny")
    _say("tiny sampled T=0")
    W = make_weights(cfg, seed=0, device="cuda")
    prompt = make_prompt(cfg)
    eng = kie.Engine(cfg, W)
    eng.prefill(prompt)
    tg, zg = eng.decode(12)
    eng.reset()
    eng.prefill(prompt)
    ts, zs = eng.decode(12, seed=5, temperature=0.0)
    np.testing.assert_array_equal(ts.cpu().numpy(), tg.cpu().numpy())
    np.testing.assert_array_equal(zs.cpu().numpy(), zg.cpu().numpy())
    pos = eng.position
    out = torch.empty(4, dtype=torch.int32, device="cuda")
    for bad in (-0.5, float("nan"), float("inf")):
        with pytest.raises(RuntimeError):
            eng.decode_sampled_into(4, 1, bad, out)
        assert eng.position == pos          # rejected before any launch
    eng.close()


def test_2b_full_vocab_sampled_draws(torch, kie):
    """Full-size model and vocabulary (32,768): a few sampled steps, each draw
    recomputed from the kernel's logits by the oracle's sampler."""
    cfg = get_config("2b")
    _say("2b sampled")
    W = make_weights(cfg, seed=0, device="cuda")
    prompt = make_prompt(cfg)
    P = len(prompt)
    eng = kie.Engine(cfg, W, max_seq=P + 16)
    eng.prefill(prompt)
    toks, z = eng.decode(6, seed=31337, temperature=0.9)
    toks, z = toks.cpu().numpy(), z.cpu().numpy()
    for i in range(len(toks)):
        keys = sample_keys(z[i], 0.9, 31337, P - 1 + i).astype(np.float64)
        order = np.argsort(-keys, kind="stable")
        if keys[order[0]] - keys[order[1]] > KEY_MARGIN * max(1.0, abs(keys[order[0]])):
            assert int(toks[i]) == int(order[0]) == sample_token(z[i], 0.9, 31337, P - 1 + i), i
        else:
            assert int(toks[i]) in (int(order[0]), int(order[1])), i
    eng.close()


# ---- top-k / top-p
from tests.parity import ABS_TOL, check_topkp_step  # noqa: E402


@pytest.mark.parametrize("name,temperature,top_k,top_p", [
    ("tiny", 1.0, 1, 1.0), ("tiny", 0.8, 5, 1.0), ("tiny", 1.2, 0, 0.9), ("tiny", 0.7, 40, 0.6),
    ("tiny", 2.0, 256, 0.97), ("2b", 1.0, 50, 0.9), ("2b", 0.6, 0, 0.95)])
def test_topkp_draws_match_the_oracle_sampler(torch, kie, name, temperature, top_k, top_p):
    """Each token is recomputed by the oracle's top-k / top-p sampler from the
    kernel's own logits (pinned unless a key or the nucleus cut is within
    float64 slack); the logits follow a teacher-forced oracle replay."""
    cfg = get_config(name, n_layers=2) if name == "2b" else get_config(name)
    _say("top-k/top-p", name, temperature, top_k, top_p)
    W = make_weights(cfg, seed=0, device="cuda")
    prompt = make_prompt(cfg)
    P = len(prompt)
    n = 16
    seed = 0xC0FFEE + top_k
    eng = kie.Engine(cfg, W, max_seq=P + n + 4)
    eng.prefill(prompt)
    toks, z = eng.decode(n, seed=seed, temperature=temperature, top_k=top_k, top_p=top_p)
    toks, z = toks.cpu().numpy(), z.cpu().numpy()
    assert eng.position == P - 1 + n
    pinned = sum(check_topkp_step(z[i], int(toks[i]), temperature, seed, P - 1 + i, top_k, top_p)
                 for i in range(n))
    assert pinned >= n - 2, pinned
    if top_k == 1:
        np.testing.assert_array_equal(toks, np.argmax(z, axis=1))     # the greedy token
    o = Oracle(cfg, weights_to_numpy(W))
    o.prefill(prompt)
    _, zo = o.decode(n, force=toks)
    assert float(np.max(np.abs(z.astype(np.float64) - zo))) <= ABS_TOL
    eng.close()


def test_topkp_is_deterministic_composable_and_validated(torch, kie):
    cfg = get_config("tiny")
    _say("top-k/top-p determinism")
    W = make_weights(cfg, seed=0, device="cuda")
    prompt = make_prompt(cfg)
    eng = kie.Engine(cfg, W)
    eng.prefill(prompt)
    t1, z1 = eng.decode(20, seed=7, temperature=1.0, top_k=30, top_p=0.8)
    eng.reset()
    eng.prefill(prompt)
    ta, _ = eng.decode(8, seed=7, temperature=1.0, top_k=30, top_p=0.8)
    tb, _ = eng.decode(12, seed=7, temperature=1.0, top_k=30, top_p=0.8)
    np.testing.assert_array_equal(np.concatenate([ta.cpu().numpy(), tb.cpu().numpy()]), t1.cpu().numpy())
    # no restriction is plain temperature sampling, bit for bit
    eng.reset()
    eng.prefill(prompt)
    tu, zu = eng.decode(20, seed=7, temperature=1.0, top_k=0, top_p=1.0)
    eng.reset()
    eng.prefill(prompt)
    ts, zs = eng.decode(20, seed=7, temperature=1.0)
    np.testing.assert_array_equal(tu.cpu().numpy(), ts.cpu().numpy())
    pos = eng.position
    out = torch.empty(4, dtype=torch.int32, device="cuda")
    for t, k, p in ((0.0, 5, 0.9), (1.0, -1, 0.9), (1.0, 257, 0.9), (1.0, 5, 0.0), (1.0, 5, 1.5),
                    (float("nan"), 5, 0.9), (1.0, 5, float("nan"))):
        with pytest.raises(RuntimeError):
            eng.decode_topkp_into(4, 1, t, k, p, out)
        assert eng.position == pos
    eng.close()
    # the staged mode refuses a restricted draw, before any launch
    g = kie.Engine(cfg, W, graph=True)
    g.prefill(prompt)
    with pytest.raises(RuntimeError):
        g.decode_topkp_into(4, 1, 1.0, 5, 0.9, out)
    g.close()
