"""Pins for the CPU oracle (no GPU).  Each test ties one oracle function to a
fact fixed outside the oracle: a closed form, an invariant, a special case,
a reduction, or an independent brute-force recompute."""
import math

import numpy as np
import pytest

import oracle
from oracle import (Oracle, argmax_first, attend, moe_ffn, moe_route, rmsnorm, rope,
                    rope_cos_sin, silu, softmax, swiglu)
from kie_synth import ModelConfig, get_config, make_prompt, make_weights, weights_to_numpy
from tests import brute


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- softmax
def test_softmax_rows_sum_to_one():
    s = _rng(1).normal(0, 3, size=(64, 257)).astype(np.float32)
    p = softmax(s)
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-6)


def test_softmax_two_point_closed_form():
    a, b = 0.3, -1.7
    p = softmax(np.array([a, b], np.float64))
    assert p[0] == pytest.approx(1.0 / (1.0 + math.exp(b - a)), rel=1e-15)
    assert p[1] == pytest.approx(1.0 / (1.0 + math.exp(a - b)), rel=1e-15)


def test_softmax_large_logits_stable():
    p = softmax(np.array([1000.0, 1000.0, -1000.0], np.float32))
    np.testing.assert_allclose(p, [0.5, 0.5, 0.0], atol=1e-7)


# -------------------------------------------------------------- attention
def test_attention_position0_is_v():
    r = _rng(2)
    for hd in (64, 80, 128):
        q = r.normal(size=hd).astype(np.float32)
        K = r.normal(size=(1, hd)).astype(np.float32)
        V = r.normal(size=(1, hd)).astype(np.float32)
        np.testing.assert_array_equal(attend(q, K, V), V[0])


def test_attention_two_keys_closed_form():
    r = _rng(3)
    hd = 128
    q, k0, k1, v0, v1 = (r.normal(size=hd) for _ in range(5))
    s0, s1 = q @ k0 / math.sqrt(hd), q @ k1 / math.sqrt(hd)
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    want = (1 - w1) * v0 + w1 * v1
    got = attend(q, np.stack([k0, k1]), np.stack([v0, v1]))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_attention_equal_scores_average():
    # q orthogonal to every key -> uniform weights -> mean of V
    hd, n = 64, 7
    q = np.zeros(hd); q[0] = 1.0
    K = _rng(4).normal(size=(n, hd)); K[:, 0] = 0.0
    V = _rng(5).normal(size=(n, hd))
    np.testing.assert_allclose(attend(q, K, V), V.mean(0), rtol=1e-12)


# ------------------------------------------------------------------- RoPE
def test_rope_position0_identity():
    v = _rng(6).normal(size=(5, 128)).astype(np.float32)
    c, s = rope_cos_sin(0, 128, 10000.0)
    np.testing.assert_array_equal(rope(v, c, s), v)


def test_rope_preserves_pair_norms():
    hd = 80
    v = _rng(7).normal(size=(3, hd))
    for p in (1, 17, 8191):
        c, s = rope_cos_sin(p, hd, 10000.0, np.float64)
        w = rope(v, c, s)
        half = hd // 2
        np.testing.assert_allclose(w[:, :half] ** 2 + w[:, half:] ** 2,
                                   v[:, :half] ** 2 + v[:, half:] ** 2, rtol=1e-12)
        np.testing.assert_allclose(np.linalg.norm(w, axis=-1), np.linalg.norm(v, axis=-1), rtol=1e-12)


def test_rope_relative_position_invariance():
    hd = 128
    r = _rng(8)
    q, k = r.normal(size=hd), r.normal(size=hd)
    def dot(m, n):
        cm, sm = rope_cos_sin(m, hd, 10000.0, np.float64)
        cn, sn = rope_cos_sin(n, hd, 10000.0, np.float64)
        return rope(q, cm, sm) @ rope(k, cn, sn)
    assert dot(5, 3) == pytest.approx(dot(105, 103), rel=1e-9)
    assert dot(700, 2) == pytest.approx(dot(1698, 1000), rel=1e-9)


def test_rope_matches_complex_rotation():
    hd, p, base = 64, 37, 10000.0
    v = _rng(9).normal(size=hd)
    half = hd // 2
    z = (v[:half] + 1j * v[half:]) * np.exp(1j * p * base ** (-2.0 * np.arange(half) / hd))
    c, s = rope_cos_sin(p, hd, base, np.float64)
    np.testing.assert_allclose(rope(v, c, s), np.concatenate([z.real, z.imag]), atol=1e-12)


def test_rope_first_pair_known_angle():
    # theta_0 = 1 for every base: the first pair turns by exactly p radians
    c, s = rope_cos_sin(3, 16, 10000.0, np.float64)
    v = np.zeros(16); v[0] = 1.0
    w = rope(v, c, s)
    assert w[0] == pytest.approx(math.cos(3.0)) and w[8] == pytest.approx(math.sin(3.0))
    assert c[-1] == pytest.approx(math.cos(3.0 * 10000.0 ** (-14.0 / 16)))


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_unit_mean_square():
    x = _rng(10).normal(0, 5, size=(4, 2560))
    y = rmsnorm(x, np.ones(2560), 0.0)
    np.testing.assert_allclose(np.mean(y * y, -1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(rmsnorm(3.7 * x, np.ones(2560), 0.0), y, rtol=1e-12)


def test_rmsnorm_constant_vector_with_eps():
    c, eps = 0.02, 1e-5
    y = rmsnorm(np.full(256, c), np.ones(256), eps)
    np.testing.assert_allclose(y, c / math.sqrt(c * c + eps), rtol=1e-12)


def test_rmsnorm_gain_is_elementwise():
    x = _rng(11).normal(size=8)
    g = np.arange(1, 9, dtype=np.float64)
    np.testing.assert_allclose(rmsnorm(x, g, 1e-5), rmsnorm(x, np.ones(8), 1e-5) * g, rtol=1e-15)


# ------------------------------------------------------------ SiLU / SwiGLU
def test_silu_closed_forms():
    a = np.linspace(-20, 20, 401)
    np.testing.assert_allclose(silu(a) - silu(-a), a, atol=1e-12)   # a*s(a) + a*s(-a) = a
    assert silu(np.array([0.0]))[0] == 0.0
    assert silu(np.array([math.log(3.0)]))[0] == pytest.approx(0.75 * math.log(3.0), rel=1e-14)


def test_swiglu_brute_force_loops():
    r = _rng(12)
    d, F = 5, 3
    h = r.normal(size=d)
    wg, wu, wd = r.normal(size=(F, d)), r.normal(size=(F, d)), r.normal(size=(d, F))
    want = np.zeros(d)
    for o in range(d):
        for f in range(F):
            g = sum(wg[f, i] * h[i] for i in range(d))
            u = sum(wu[f, i] * h[i] for i in range(d))
            want[o] += wd[o, f] * (g / (1 + math.exp(-g))) * u
    np.testing.assert_allclose(swiglu(h, wg, wu, wd), want, rtol=1e-12)
    np.testing.assert_allclose(swiglu(h[None], wg, wu, wd)[0], want, rtol=1e-12)


# ------------------------------------------------------------------ argmax
def test_argmax_ties_pick_lowest_index():
    z = np.zeros(100, np.float32)
    z[[7, 42, 99]] = 3.0
    assert argmax_first(z) == 7
    z[3] = np.nextafter(np.float32(3.0), np.float32(0))
    assert argmax_first(z) == 7


# --------------------------------------------------------------------- MoE
def test_moe_zero_router_uniform_and_lowest_ids():
    pi, sel = moe_route(np.zeros(64, np.float32), 6)
    np.testing.assert_allclose(pi, 1.0 / 64, rtol=1e-6)
    assert list(sel) == [0, 1, 2, 3, 4, 5]


def test_moe_route_order_and_unnormalised_weights():
    r = np.array([0.0, 2.0, 1.0, 2.0, -1.0])
    pi, sel = moe_route(r, 3)
    assert list(sel) == [1, 3, 2]                      # tie 1 vs 3 -> lower id first
    e = np.exp(r - r.max())
    np.testing.assert_allclose(pi, e / e.sum(), rtol=1e-15)
    assert pi[sel].sum() < 1.0                          # not renormalised


def test_moe_single_expert_reduces_to_dense():
    r = _rng(13)
    d, F = 16, 24
    h = r.normal(size=d)
    g, u, dn = r.normal(size=(1, F, d)), r.normal(size=(1, F, d)), r.normal(size=(1, d, F))
    y, sel = moe_ffn(h, r.normal(size=(1, d)), lambda e: (g[e], u[e], dn[e]), 1, 1, 0)
    np.testing.assert_allclose(y, swiglu(h, g[0], u[0], dn[0]), rtol=1e-15)
    assert list(sel) == [0]


def test_moe_renormalised_weights_sum_to_one():
    # every routed expert computes the same function f, so the routed part is
    # (sum of the weights) * f: exactly f when renormalised, sum(pi_sel) * f otherwise
    r = _rng(15)
    d, F = 8, 6
    h = r.normal(size=d)
    same = (r.normal(size=(F, d)), r.normal(size=(F, d)), r.normal(size=(d, F)))
    router = r.normal(size=(7, d))
    f = swiglu(h, *same)
    y, sel = moe_ffn(h, router, lambda e: same, 7, 3, 0, renorm=True)
    np.testing.assert_allclose(y, f, rtol=1e-13)
    pi, _ = moe_route(router @ h, 3)
    y0, _ = moe_ffn(h, router, lambda e: same, 7, 3, 0)
    np.testing.assert_allclose(y0, pi[sel].sum() * f, rtol=1e-13)


def test_moe_renormalised_with_every_expert_selected_is_plain_softmax():
    r = _rng(16)
    d, F = 8, 5
    h = r.normal(size=d)
    ex = [(r.normal(size=(F, d)), r.normal(size=(F, d)), r.normal(size=(d, F))) for _ in range(5)]
    router = r.normal(size=(4, d))
    y1, _ = moe_ffn(h, router, lambda e: ex[e], 4, 4, 1, renorm=True)
    y0, _ = moe_ffn(h, router, lambda e: ex[e], 4, 4, 1)
    np.testing.assert_allclose(y1, y0, rtol=1e-12)


def test_moe_shared_only():
    r = _rng(14)
    d, F = 8, 4
    h = r.normal(size=d)
    ex = [(r.normal(size=(F, d)), r.normal(size=(F, d)), r.normal(size=(d, F))) for _ in range(5)]
    # router logits of -inf-like magnitude never matter to the shared experts
    y, _ = moe_ffn(h, np.zeros((3, d)), lambda e: ex[e], 3, 1, 2)
    want = swiglu(h, *ex[3]) + swiglu(h, *ex[4]) + (1.0 / 3) * swiglu(h, *ex[0])
    np.testing.assert_allclose(y, want, rtol=1e-13)


# ---------------------------------------------------- whole decoder, brute force
SMALL = ModelConfig("small", n_layers=2, d_model=32, n_heads=4, n_kv_heads=4, head_dim=8,
                    ffn_hidden=48, vocab_in=61, vocab_out=53, prompt_len=6, n_decode=5)
SMALL_GQA = SMALL.with_(name="small_gqa", n_kv_heads=2)
SMALL_MOE = SMALL.with_(name="small_moe", ffn_hidden=0, n_experts=5, top_k=2,
                        n_shared_experts=1, expert_hidden=12)


def _np_weights(cfg, seed=0, std=0.02):
    return weights_to_numpy(make_weights(cfg, seed=seed, std=std))


SMALL_MOE_RENORM = SMALL_MOE.with_(name="small_moe_renorm", moe_renorm=True)


@pytest.mark.parametrize("cfg", [SMALL, SMALL_GQA, SMALL_MOE, SMALL_MOE_RENORM], ids=lambda c: c.name)
def test_decoder_matches_brute_force_recompute(cfg):
    # std 0.3 makes attention and routing far from uniform, so a wrong index
    # or sign shows up in the logits
    W = _np_weights(cfg, seed=3, std=0.3)
    prompt = make_prompt(cfg, seed=1)
    o = Oracle(cfg, W, dtype=np.float64)
    o.prefill(prompt)
    toks, logits = o.decode(cfg.n_decode)
    seq = list(prompt)
    for i in range(cfg.n_decode):
        want, chosen = brute.last_logits(cfg, W, seq, return_experts=True)
        np.testing.assert_allclose(logits[i], want, rtol=1e-9, atol=1e-11)
        if cfg.n_experts:
            np.testing.assert_array_equal(o.expert_log[i], np.array(chosen))
        assert toks[i] == int(np.argmax(want))
        seq.append(int(toks[i]))


def test_batched_prefill_equals_sequential():
    cfg = get_config("tiny")
    W = _np_weights(cfg)
    prompt = make_prompt(cfg)
    a = Oracle(cfg, W)
    b = Oracle(cfg, W)
    a.prefill(prompt, batched=True)
    b.prefill(prompt, batched=False)
    P = len(prompt)
    for l in range(cfg.n_layers):
        np.testing.assert_allclose(a.K[l][:, :P - 1], b.K[l][:, :P - 1], atol=1e-5, rtol=1e-5)
        np.testing.assert_allclose(a.V[l][:, :P - 1], b.V[l][:, :P - 1], atol=1e-5, rtol=1e-5)
    ta, za = a.decode(8)
    tb, zb = b.decode(8)
    np.testing.assert_allclose(za, zb, atol=1e-4)


def test_moe_routing_record_is_per_position_and_prefill_independent():
    """The routing record is keyed by position; batched prefill records the
    same experts (and router logits, to rounding) as running the prompt
    through the one-token step, and each decode step adds its position."""
    cfg = SMALL_MOE.with_(prompt_len=9)
    W = _np_weights(cfg, std=0.3)
    prompt = make_prompt(cfg)
    a = Oracle(cfg, W)
    b = Oracle(cfg, W)
    a.prefill(prompt, batched=True)
    b.prefill(prompt, batched=False)
    P = len(prompt)
    assert sorted(a.route) == sorted(b.route) == list(range(P - 1))
    for p in range(P - 1):
        np.testing.assert_array_equal(a.route[p][0], b.route[p][0])
        np.testing.assert_allclose(a.route[p][1], b.route[p][1], atol=1e-5)
        assert a.route[p][0].shape == (cfg.n_layers, cfg.top_k)
    for l in range(cfg.n_layers):
        np.testing.assert_allclose(a.K[l][:, :P - 1], b.K[l][:, :P - 1], atol=1e-5, rtol=1e-5)
        np.testing.assert_allclose(a.V[l][:, :P - 1], b.V[l][:, :P - 1], atol=1e-5, rtol=1e-5)
    np.testing.assert_allclose(a.decode(2)[1], b.decode(2)[1], atol=1e-5, rtol=1e-5)
    a.reset(); a.prefill(prompt, batched=True)
    a.decode(3)
    assert sorted(a.route) == list(range(P + 2))
    for i in range(3):
        np.testing.assert_array_equal(a.route[P - 1 + i][0], a.expert_log[i])


def test_routing_comparison_accepts_only_near_ties():
    from tests.parity import compare_routing
    r = np.array([[[5.0, 4.0, 3.0, 2.9995, 1.0]]])          # 3rd/4th logits 5e-4 apart
    ok = np.array([[[0, 1, 2]]])
    assert compare_routing(ok, ok, r, 3) == []
    assert compare_routing(np.array([[[0, 1, 3]]]), ok, r, 3) == [0]   # near-tie swap
    with pytest.raises(AssertionError):
        compare_routing(np.array([[[0, 1, 4]]]), ok, r, 3)         # not a near tie
    with pytest.raises(AssertionError):
        compare_routing(np.array([[[1, 0, 2]]]), ok, r, 3)         # order of clear winners
    r2 = np.array([[[5.0, 4.9995, 3.0, 1.0, 0.0]]])
    assert compare_routing(np.array([[[1, 0, 2]]]), ok, r2, 3) == []   # order of tied pair
    # a near-tie flip in layer 0 changes layer 1's input: layer 1 is not compared
    r3 = np.concatenate([r, np.array([[[9.0, 0.0, 0.0, 0.0, 8.0]]])], axis=1)
    both = np.array([[[0, 1, 2], [0, 4, 1]]])
    where = {}
    assert compare_routing(np.array([[[0, 1, 3], [1, 2, 3]]]), both, r3, 3, where) == [0]
    assert where == {0: 0}


def test_gqa_equals_mha_with_repeated_kv_rows():
    cfg = SMALL_GQA
    W = _np_weights(cfg, seed=5, std=0.3)
    G = cfg.n_heads // cfg.n_kv_heads
    hd = cfg.head_dim
    mha = cfg.with_(name="mha", n_kv_heads=cfg.n_heads)
    W2 = {k: v for k, v in W.items()}
    W2["layers"] = []
    for lw in W["layers"]:
        lw2 = dict(lw)
        for nm in ("wk", "wv"):
            blocks = lw[nm].reshape(cfg.n_kv_heads, hd, cfg.d_model)
            lw2[nm] = np.repeat(blocks, G, axis=0).reshape(cfg.n_heads * hd, cfg.d_model)
        W2["layers"].append(lw2)
    prompt = make_prompt(cfg, seed=2)
    a, b = Oracle(cfg, W, np.float64), Oracle(mha, W2, np.float64)
    a.prefill(prompt); b.prefill(prompt)
    np.testing.assert_allclose(a.decode(4)[1], b.decode(4)[1], rtol=1e-12, atol=1e-14)


def test_force_with_own_tokens_is_free_running_and_composable():
    cfg = get_config("tiny")
    W = _np_weights(cfg)
    prompt = make_prompt(cfg)
    a = Oracle(cfg, W); a.prefill(prompt)
    ta, za = a.decode(10)
    b = Oracle(cfg, W); b.prefill(prompt)
    tb, zb = b.decode(10, force=ta)
    np.testing.assert_array_equal(ta, tb)
    np.testing.assert_array_equal(za, zb)
    c = Oracle(cfg, W); c.prefill(prompt)
    t1, z1 = c.decode(4)
    t2, z2 = c.decode(6)
    np.testing.assert_array_equal(np.concatenate([t1, t2]), ta)
    np.testing.assert_array_equal(np.concatenate([z1, z2]), za)
    assert c.pos == len(prompt) - 1 + 10


def test_state_errors():
    cfg = SMALL
    W = _np_weights(cfg)
    o = Oracle(cfg, W)
    with pytest.raises(ValueError):
        o.decode(1)                          # no prompt yet
    o.prefill([1, 2, 3])
    with pytest.raises(ValueError):
        o.prefill([1, 2])                    # not fresh
    with pytest.raises(ValueError):
        o.decode(cfg.kv_capacity)            # overflow
    with pytest.raises(ValueError):
        Oracle(cfg, W).prefill([cfg.vocab_in])


def test_kv_fp16_switch_is_close():
    cfg = get_config("tiny")
    W = _np_weights(cfg)
    prompt = make_prompt(cfg)
    a = Oracle(cfg, W); a.prefill(prompt)
    b = Oracle(cfg, W, kv_fp16=True); b.prefill(prompt)
    za, zb = a.decode(4)[1], b.decode(4)[1]
    assert np.max(np.abs(za - zb)) < 2e-3


def test_kv_fp16_switch_drift_is_bounded_for_moe():
    # The MoE GPU comparisons run the oracle with an fp16 KV cache (the
    # kernel's cache precision), so that both sides take each routing
    # decision from the same rounded rows.  That switch must itself stay close
    # to the fp32-KV definition: on a narrow MoE (8 experts, top 2 + 1
    # shared), teacher-forced on the fp32 oracle's own tokens, the logits
    # move by far less than the parity bar and no routing decision changes.
    cfg = get_config("moe", n_layers=2, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64,
                     vocab_in=4096, vocab_out=4096, n_experts=8, top_k=2, n_shared_experts=1,
                     expert_hidden=128, prompt_len=64, n_decode=24)
    W = _np_weights(cfg)
    prompt = make_prompt(cfg)
    a = Oracle(cfg, W)
    a.prefill(prompt)
    toks, za = a.decode(cfg.n_decode)
    b = Oracle(cfg, W, kv_fp16=True)
    b.prefill(prompt)
    _, zb = b.decode(cfg.n_decode, force=toks)
    drift = np.abs(za.astype(np.float64) - zb)
    assert drift.max() < 2e-3, drift.max()
    assert np.all(drift.max(axis=1) < 1e-3 * (za.max(axis=1) - za.min(axis=1)))
    for q in range(len(prompt) - 1 + cfg.n_decode):
        np.testing.assert_array_equal(a.route[q][0], b.route[q][0])


@pytest.mark.slow
def test_logit_statistics_at_2b_width():
    # logits = W_lm rms(x) with W_lm ~ N(0, 0.02) and unit-gain rms -> std ~ 0.02*sqrt(d)
    cfg = get_config("2b").with_(name="2b_2layer", n_layers=2, vocab_in=4096, vocab_out=4096,
                                 prompt_len=4, n_decode=2)
    W = _np_weights(cfg)
    o = Oracle(cfg, W)
    o.prefill(make_prompt(cfg))
    z = o.decode(2)[1]
    want = 0.02 * math.sqrt(cfg.d_model)
    assert abs(z.std() / want - 1.0) < 0.2
