"""Each decode stage in isolation against float64 (kie_debug_stage).

On a prefilled handle the next decode step runs one stage at a time; each
stage's output is compared with a float64 computation from the inputs that
stage actually consumed (the previous stage's output as the kernel wrote
it), so an error is pinned to its stage: RMSNorm with non-trivial gains and
the Q/K/V products, RoPE and the fp16 K/V append, split-K attention with its
merge (several splits and one), the O product and residual, gate/up with
SwiGLU, down and residual, the MoE router, routing and experts, the final
norm with lm_head, and the argmax.  The step the stages build must also equal
an ordinary decode step of the persistent kernel, bit for bit.
"""
import sys

import numpy as np
import pytest

from kie_synth import get_config, make_prompt, make_weights, weights_to_numpy
from oracle.decoder import argmax_first

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


def f64(a):
    return np.asarray(a, dtype=np.float64)


def round24(x):
    """fp32 values as they cross between workgroups: the top 24 bits of the
    pattern, rounded to nearest even."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7F + ((b >> 8) & 1)) >> 8) << 8
    return (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)


def rms(x, g, eps):
    x = f64(x)
    return x / np.sqrt(np.mean(x * x) + eps) * f64(g)


def close(got, want, scale, rel=2e-5, what=""):
    """|got - want| within rel of the sum of |terms| (scale) per element."""
    err = np.abs(f64(got) - want)
    bound = rel * f64(scale) + 1e-30
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, (what, int(bad[0]), float(err[bad[0]]), float(bound[bad[0]]))


def rope(v, pos, base, hd):
    """Rotate-half RoPE with the runtime's table (float64 angle, cos/sin rounded to fp32)."""
    half = hd // 2
    j = np.arange(half)
    th = np.power(float(base), -2.0 * j / hd)
    c = np.cos(pos * th).astype(np.float32).astype(np.float64)
    s = np.sin(pos * th).astype(np.float32).astype(np.float64)
    v = f64(v)
    a, b = v[..., :half], v[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def _random_gains(torch, W, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for lw in W["layers"]:
        for k in ("attn_norm", "ffn_norm"):
            lw[k] = (1.0 + 0.5 * torch.randn(lw[k].shape, generator=g, device="cuda")).half()
    W["final_norm"] = (1.0 + 0.5 * torch.randn(W["final_norm"].shape, generator=g, device="cuda")).half()
    return W


def _check_attention(eng, cfg, layer, pos, qkv, o):
    H, nkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    qd, kd = H * hd, nkv * hd
    q = rope(qkv[:qd].reshape(H, hd), pos, cfg.rope_base, hd)
    k = rope(qkv[qd:qd + kd].reshape(nkv, hd), pos, cfg.rope_base, hd)
    v = qkv[qd + kd:].reshape(nkv, hd).astype(np.float32)
    K, V = eng.read_kv(layer, 0, pos + 1)                     # fp16 [nkv][pos + 1][hd]
    # the appended row: fp16 of the rotated key within half an fp16 ulp, the
    # value row exactly fp16 of the kernel's fp32 value
    kn = f64(K[:, pos])
    ulp = np.spacing(np.abs(k).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(kn - k) <= 0.5 * ulp + 1e-6 * np.abs(k)), "appended K row"
    assert np.array_equal(V[:, pos].view(np.uint16), v.astype(np.float16).view(np.uint16)), "appended V row"
    g = H // nkv
    want = np.empty((H, hd))
    scale = np.empty((H, hd))
    for h in range(H):
        Kh, Vh = f64(K[h // g]), f64(V[h // g])
        s = Kh @ q[h] / np.sqrt(hd)
        a = np.exp(s - s.max())
        a /= a.sum()
        want[h] = a @ Vh
        scale[h] = a @ np.abs(Vh)
    # o crossed as 24-bit values (relative 2^-16) after fp32 accumulation
    close(o, want.reshape(-1), scale.reshape(-1) + np.abs(want.reshape(-1)), rel=4e-5, what="attention")


@pytest.mark.parametrize("prompt_len,shape", [
    (600, {}), (40, {}),
    # grouped query heads (4 per KV head): the matrix-core attention
    (600, dict(n_heads=8, n_kv_heads=2, head_dim=32)),
    (300, dict(n_heads=16, n_kv_heads=4, head_dim=80)),
], ids=["mha600", "mha40", "gqa4_hd32", "gqa4_hd80"])
def test_dense_stages_match_float64(torch, kie, prompt_len, shape):
    """tiny widths; at position 599 the attention runs 5 splits and a merge,
    at position 39 one split; the grouped shapes take the matrix-core form."""
    cfg = get_config("tiny", **shape)
    _say("stages dense", prompt_len, shape)
    W = _random_gains(torch, make_weights(cfg, seed=5, device="cuda"), 9)
    Wn = weights_to_numpy(W)
    prompt = make_prompt(cfg, seed=2, length=prompt_len)
    pos, tok = prompt_len - 1, int(prompt[-1])
    eng = kie.Engine(cfg, W, max_seq=prompt_len + 8)
    eng.prefill_batched(prompt)
    eps = cfg.rms_eps
    x = f64(Wn["tok_emb"][tok].astype(np.float32))
    for l in range(cfg.n_layers):
        lw = Wn["layers"][l]
        wqkv = f64(np.concatenate([lw["wq"], lw["wk"], lw["wv"]]))
        eng.debug_stage("qkv", l)
        qkv = eng.debug_read_act("qkv", l)
        xin = x if l == 0 else f64(round24(x))         # later layers read x as 24-bit values
        h = rms(xin, lw["attn_norm"], eps)
        close(qkv, wqkv @ h, np.abs(wqkv) @ np.abs(h), what=f"qkv {l}")
        eng.debug_stage("attention", l)
        o = eng.debug_read_act("o", l)
        _check_attention(eng, cfg, l, pos, qkv, o)
        eng.debug_stage("o", l)
        xa = eng.debug_read_act("x_attn", l)
        wo = f64(lw["wo"])
        close(xa, x + wo @ f64(o), np.abs(wo) @ np.abs(f64(o)) + np.abs(x), what=f"o {l}")
        eng.debug_stage("gateup", l)
        u = eng.debug_read_act("u", l)
        h2 = rms(round24(xa), lw["ffn_norm"], eps)
        wg, wu = f64(lw["w_gate"]), f64(lw["w_up"])
        gg, uu = wg @ h2, wu @ h2
        silu = gg / (1.0 + np.exp(-gg))
        want_u = silu * uu
        sc = (np.abs(wg) @ np.abs(h2)) * np.abs(uu) + np.abs(silu) * (np.abs(wu) @ np.abs(h2)) + np.abs(want_u)
        close(u, want_u, sc, rel=4e-5, what=f"gateup {l}")
        eng.debug_stage("down", l)
        xd = eng.debug_read_act("x", l)
        wd = f64(lw["w_down"])
        close(xd, f64(xa) + wd @ f64(u), np.abs(wd) @ np.abs(f64(u)) + np.abs(f64(xa)), what=f"down {l}")
        x = f64(xd)
    eng.debug_stage("lm_head", 0)
    z = eng.debug_read_act("logits")
    t = eng.debug_read_act("token")
    hf = rms(x, Wn["final_norm"], eps)
    wl = f64(Wn["lm_head"])
    close(z, wl @ hf, np.abs(wl) @ np.abs(hf), what="lm_head")
    assert t == argmax_first(z)
    # the same step as one persistent launch: identical logits and token
    toks, zd = eng.decode(1)
    assert int(toks[0]) == t
    assert np.array_equal(zd[0].cpu().numpy().view(np.uint32), z.view(np.uint32))
    eng.close()


def test_moe_stages_match_float64(torch, kie):
    cfg = get_config("moe", n_layers=2)
    _say("stages moe")
    W = _random_gains(torch, make_weights(cfg, seed=6, device="cuda"), 10)
    Wn = weights_to_numpy(W)
    prompt = make_prompt(cfg, seed=3, length=40)
    pos, tok = 39, int(prompt[-1])
    eng = kie.Engine(cfg, W, max_seq=48)
    eng.prefill_batched(prompt)
    eps, E, K, S, Fe = cfg.rms_eps, cfg.n_experts, cfg.top_k, cfg.n_shared_experts, cfg.expert_hidden
    x = f64(Wn["tok_emb"][tok].astype(np.float32))
    routed = []
    for l in range(cfg.n_layers):
        lw = Wn["layers"][l]
        eng.debug_stage("qkv", l)
        qkv = eng.debug_read_act("qkv", l)
        eng.debug_stage("attention", l)
        _check_attention(eng, cfg, l, pos, qkv, eng.debug_read_act("o", l))
        eng.debug_stage("o", l)
        xa = f64(eng.debug_read_act("x_attn", l))
        eng.debug_stage("router", l)
        r = eng.debug_read_act("router", l)
        h2 = rms(xa, lw["ffn_norm"], eps)                # the router and experts read fp32 x
        wr = f64(lw["router"])
        close(r, wr @ h2, np.abs(wr) @ np.abs(h2), what=f"router {l}")
        eng.debug_stage("moe_gateup", l)
        u = eng.debug_read_act("u", l)
        # routing from the kernel's own router logits: softmax, top-k by
        # probability with ties to the lower id, weights not renormalised
        rl = f64(r.astype(np.float32))
        p = np.exp(rl - rl.max())
        p /= p.sum()
        ids = sorted(range(E), key=lambda e: (-r[e], e))[:K]
        routed.append(ids)
        slots = [(e, p[e]) for e in ids] + [(E + a, 1.0) for a in range(S)]
        want_u, sc = [], []
        for e, wgt in slots:
            ge, ue = f64(lw["e_gate"][e]) @ h2, f64(lw["e_up"][e]) @ h2
            silu = ge / (1.0 + np.exp(-ge))
            want_u.append(wgt * silu * ue)
            sc.append(wgt * ((np.abs(f64(lw["e_gate"][e])) @ np.abs(h2)) * np.abs(ue)
                             + np.abs(silu) * (np.abs(f64(lw["e_up"][e])) @ np.abs(h2))) + np.abs(wgt * silu * ue))
        close(u, np.concatenate(want_u), np.concatenate(sc), rel=5e-5, what=f"moe gateup {l}")
        eng.debug_stage("moe_down", l)
        xd = eng.debug_read_act("x", l)
        want = f64(xa).copy()
        sc = np.abs(f64(xa))
        for a, (e, _) in enumerate(slots):
            wd = f64(lw["e_down"][e])
            ua = f64(u[a * Fe:(a + 1) * Fe])
            want += wd @ ua
            sc += np.abs(wd) @ np.abs(ua)
        close(xd, want, sc, what=f"moe down {l}")
        x = f64(xd)
    eng.debug_stage("lm_head", 0)
    z = eng.debug_read_act("logits")
    assert eng.debug_read_act("token") == argmax_first(z)
    toks, zd = eng.decode(1)
    assert np.array_equal(zd[0].cpu().numpy().view(np.uint32), z.view(np.uint32))
    # the routing record of that position: the experts the stages used
    assert eng.expert_ids(pos, pos + 1)[0].tolist() == routed
    eng.close()


def test_stage_entry_checks_its_state(torch, kie):
    cfg = get_config("tiny")
    W = make_weights(cfg, seed=0, device="cuda")
    eng = kie.Engine(cfg, W)
    with pytest.raises(RuntimeError):
        eng.debug_stage("qkv", 0)                      # no pending token
    eng.prefill(make_prompt(cfg))
    with pytest.raises(RuntimeError):
        eng.debug_stage("o", 0)                        # no open step
    eng.debug_stage("qkv", 0)
    with pytest.raises(RuntimeError):
        eng.debug_stage("router", 0)                   # a dense model has none
    with pytest.raises(RuntimeError):
        eng.debug_stage("qkv", cfg.n_layers)           # layer out of range
    with pytest.raises(RuntimeError):
        eng.debug_read_act("o", 0)                     # not written by this step yet
    eng.close()
