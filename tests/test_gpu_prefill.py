"""Batched prefill (kie_prefill_batched) on the GPU against the oracle.

The matrix-core product (kie_debug_gemm) is checked element by element
against float64 numpy on the same fp16 weights and fp32 activations; the
whole batched prefill is checked through the K/V rows it writes (against
the oracle's cache, with the bar used for the persistent kernel's prefill)
and through the decode that continues from it (the logit bar of the
decode tests, teacher forced)."""
import numpy as np
import pytest

from kie_synth import get_config, make_prompt, make_weights, weights_to_numpy
from tests.parity import compare_steps
from tests.test_gpu_parity import _check_kv, _moe_check, _oracle_replay, _say

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("m,n,k,acc", [(1, 64, 32, False), (5, 100, 64, True), (64, 64, 2560, False),
                                       (130, 200, 2560, True), (77, 2560, 6912, False),
                                       (513, 384, 864, True), (2048, 2560, 2560, False),
                                       (2100, 2100, 96, True)])
def test_gemm_matches_float64(torch, kie, m, n, k, acc):
    """Tiles that cover the 64 x 64 block, ragged edges in m and n, the
    accumulate form, and the inner sizes of the workloads, up to a full
    2048-position chunk of the long-context shape."""
    _say("gemm", m, n, k, acc)
    g = torch.Generator(device="cuda").manual_seed(m * 7 + n * 3 + k)
    w = (torch.randn(n, k, device="cuda", generator=g) * 0.02).half()
    a = torch.randn(m, k, device="cuda", generator=g) * 3.0
    c0 = torch.randn(m, n, device="cuda", generator=g) if acc else None
    c = kie.debug_gemm(w, a, c0.clone() if acc else None)
    torch.cuda.synchronize()
    w64 = w.float().cpu().numpy().astype(np.float64)
    a64 = a.cpu().numpy().astype(np.float64)
    ref = a64 @ w64.T
    if acc:
        ref += c0.cpu().numpy().astype(np.float64)
    bound = np.abs(a64) @ np.abs(w64).T
    err = np.abs(c.cpu().numpy().astype(np.float64) - ref)
    # fp32 accumulation over k terms plus the hi/lo representation (2^-22)
    tol = 1e-5 * bound + 1e-5 * (np.abs(ref) if acc else 0.0) + 1e-7
    assert np.all(err <= tol), f"worst excess {float(np.max(err - tol)):.3e}, worst err {float(err.max()):.3e}"


PREFILL_CASES = {
    # name: (workload, overrides, decode steps)
    "tiny": ("tiny", {}, 64),
    "gqa2_narrow": ("tiny", dict(n_heads=8, n_kv_heads=4, head_dim=32, prompt_len=80), 16),
    # head sizes whose value columns only partly fill their last 32-wide tile (16, 48, 112)
    "hd16_gqa2": ("tiny", dict(n_heads=8, n_kv_heads=4, head_dim=16, prompt_len=150), 16),
    "hd48_gqa2": ("tiny", dict(n_heads=4, n_kv_heads=2, head_dim=48, prompt_len=150), 16),
    "hd112": ("tiny", dict(n_heads=4, n_kv_heads=4, head_dim=112, prompt_len=150), 16),
    # grouped-query attention 32 x 80 over 8 KV heads, a 1200-position prompt
    "longctx_2l_1200": ("longctx", dict(n_layers=2, prompt_len=1200), 8),
    # a full first chunk of 2048 positions, then a ragged second one
    "longctx_2l_2150": ("longctx", dict(n_layers=2, prompt_len=2150), 8),
    # a narrow dense model over two chunks of 2048 positions
    "tiny_2chunks": ("tiny", dict(prompt_len=2300), 16),
    # 3 heads x 128, FFN 864, 4096-row lm_head
    "tp8share_3l": ("tp8share", dict(n_layers=3, prompt_len=96), 16),
    # 64 routed experts (top 6) + 2 shared, hidden 1408: grouped per-expert products
    "moe_2l": ("moe", dict(n_layers=2, prompt_len=48), 24),
    # a narrow MoE over a prompt of two chunks, plain and renormalised weights
    "moe_narrow_2chunks": ("moe", dict(n_layers=2, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64,
                                       vocab_in=4096, vocab_out=4096, n_experts=8, top_k=2,
                                       n_shared_experts=1, expert_hidden=128, prompt_len=2200), 16),
    "moe_narrow_renorm": ("moe", dict(n_layers=2, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64,
                                      vocab_in=4096, vocab_out=4096, n_experts=8, top_k=2,
                                      n_shared_experts=1, expert_hidden=128, prompt_len=64,
                                      moe_renorm=True), 16),
}


@pytest.mark.parametrize("key", sorted(PREFILL_CASES))
def test_prefill_batched_matches_oracle(torch, kie, key):
    name, over, n = PREFILL_CASES[key]
    cfg = get_config(name, **over)
    _say("batched prefill", key)
    W = make_weights(cfg, seed=0, device="cuda")
    prompt = make_prompt(cfg)
    P = len(prompt)
    eng = kie.Engine(cfg, W)
    eng.prefill_batched(prompt)
    assert eng.position == P - 1
    toks, z = eng.decode(n)
    torch.cuda.synchronize()
    toks = toks.cpu().numpy()
    z = z.cpu().numpy()
    o, zo = _oracle_replay(cfg, weights_to_numpy(W), prompt, toks)
    # MoE: the routing of every prompt and decode position against the
    # oracle's (an accepted near-tie excuses that position above layer 0)
    tied = _moe_check(eng, o, cfg, range(P - 1 + n)) if cfg.is_moe else []
    rep = compare_steps(z, toks, zo, skip=[q - (P - 1) for q in tied if q >= P - 1])
    _say(key, rep, "routing near-ties at positions", tied)
    assert rep["pinned"] >= max(4, n // 4)
    _check_kv(eng, o, range(cfg.n_layers), [(0, min(P - 1, 520)), (2040, 2056), (max(0, P - 40), P - 1 + n)]
              if P > 2100 else [(0, min(P - 1, 520)), (max(0, P - 40), P - 1 + n)], exclude=tied)
    eng.close()


def test_prefill_batched_agrees_with_persistent_prefill(torch, kie):
    """Both prefills write the same cache up to fp32 rounding order, so the
    greedy tokens of the decode that follows agree wherever the logits are
    not near a tie, and the logits stay within the decode bar of each other."""
    cfg = get_config("tiny")
    W = make_weights(cfg, seed=0, device="cuda")
    prompt = make_prompt(cfg)
    a = kie.Engine(cfg, W)
    a.prefill(prompt)
    ta, za = a.decode(32)
    b = kie.Engine(cfg, W)
    b.prefill_batched(prompt)
    tb, zb = b.decode(32)
    torch.cuda.synchronize()
    za, zb = za.cpu().numpy(), zb.cpu().numpy()
    ta, tb = ta.cpu().numpy(), tb.cpu().numpy()
    first = int(np.argmax(ta != tb)) if np.any(ta != tb) else len(ta)
    assert np.max(np.abs(za[:first] - zb[:first])) <= 2e-3
    for l in range(cfg.n_layers):
        ka, va = a.read_kv(l, 0, len(prompt) - 1)
        kb, vb = b.read_kv(l, 0, len(prompt) - 1)
        assert np.max(np.abs(ka.astype(np.float64) - kb.astype(np.float64))) <= 1e-2
        assert np.max(np.abs(va.astype(np.float64) - vb.astype(np.float64))) <= 1e-2
    a.close()
    b.close()


def test_prefill_batched_at_full_capacity(torch, kie):
    """A prompt that fills the cache but for the pending position: one
    decode step writes the last row, the next overflows."""
    cfg = get_config("tiny")
    W = make_weights(cfg, seed=0, device="cuda")
    prompt = make_prompt(cfg)
    P = len(prompt)
    e = kie.Engine(cfg, W, max_seq=P)
    e.prefill_batched(prompt)
    t, z = e.decode(1)
    torch.cuda.synchronize()
    assert e.position == P
    o, zo = _oracle_replay(cfg.with_(max_seq=P), weights_to_numpy(W), prompt, t.cpu().numpy())
    compare_steps(z.cpu().numpy(), t.cpu().numpy(), zo)
    _check_kv(e, o, (0, 1), [(P - 8, P)])
    with pytest.raises(kie.KieError) as ei:
        e.decode(1)
    assert ei.value.status == "KIE_ERR_CONTEXT_OVERFLOW"
    e.close()


def test_prefill_batched_then_staged_graph_decode(torch, kie):
    """The staged (hipGraph) mode decodes from the state a batched prefill
    leaves, and matches the persistent kernel decoding from it bit for bit."""
    cfg = get_config("tiny")
    W = make_weights(cfg, seed=0, device="cuda")
    prompt = make_prompt(cfg)
    a = kie.Engine(cfg, W)
    a.prefill_batched(prompt)
    ta, za = a.decode(24)
    b = kie.Engine(cfg, W, graph=True)
    b.prefill_batched(prompt)
    tb, zb = b.decode(24)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ta.cpu().numpy(), tb.cpu().numpy())
    np.testing.assert_array_equal(za.cpu().numpy(), zb.cpu().numpy())
    a.close()
    b.close()


def test_prefill_batched_rejects_unsupported_shape_and_bad_state(torch, kie):
    cfg = get_config("tiny", n_heads=4, head_dim=8, n_kv_heads=4, d_model=256)   # head_dim % 16 != 0
    W = make_weights(cfg, seed=0, device="cuda")
    e = kie.Engine(cfg, W)
    with pytest.raises(kie.KieError) as ei:
        e.prefill_batched(make_prompt(cfg))
    assert ei.value.status == "KIE_ERR_UNSUPPORTED"
    e.close()
    cfg = get_config("tiny")
    W = make_weights(cfg, seed=0, device="cuda")
    e = kie.Engine(cfg, W)
    e.prefill_batched([1, 2, 3])
    with pytest.raises(kie.KieError) as ei:
        e.prefill_batched([1, 2, 3])
    assert ei.value.status == "KIE_ERR_BAD_STATE"
    e.reset()
    e.prefill_batched([5])                 # one token: nothing to run, it becomes pending
    assert e.position == 0
    t, _ = e.decode(2)
    assert t.shape[0] == 2
    e.close()
