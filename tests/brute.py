"""Brute-force float64 decoder used only to pin the oracle.

Written independently of ``oracle/``: every prefix is recomputed from
scratch (no KV cache), attention is an explicit loop over keys, the rotary
embedding is complex multiplication by exp(i p theta_j), the sigmoid is
0.5 (1 + tanh(a/2)), and routing sorts expert ids by (-probability, id).
Only tiny shapes are feasible.
"""
from __future__ import annotations

import math

import numpy as np


def _f(a):
    return np.asarray(a, dtype=np.float64)


def _norm(v, g, eps):
    d = v.shape[0]
    ms = float(np.dot(v, v)) / d
    return v * (1.0 / math.sqrt(ms + eps)) * _f(g)


def _rotary(u, p, base):
    hd = u.shape[0]
    half = hd // 2
    z = u[:half] + 1j * u[half:]
    theta = np.array([base ** (-2.0 * j / hd) for j in range(half)])
    z = z * np.exp(1j * p * theta)
    return np.concatenate([z.real, z.imag])


def _sigmoid(a):
    return 0.5 * (1.0 + np.tanh(0.5 * a))


def _mv(w, x):
    # explicit row-major [out][in] product, one output per row
    w = _f(w)
    return np.array([float(np.dot(w[r], x)) for r in range(w.shape[0])])


def _swiglu(h, wg, wu, wd):
    g = _mv(wg, h)
    u = _mv(wu, h)
    return _mv(wd, g * _sigmoid(g) * u)


def last_logits(cfg, W, seq, return_experts=False):
    """Logits of the last position of ``seq`` and, for MoE, the selected experts
    per layer at that position."""
    L, H, nkv, hd = cfg.n_layers, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    G = H // nkv
    eps = cfg.rms_eps
    n = len(seq)
    X = [_f(W["tok_emb"][t]) for t in seq]
    chosen = []
    for l in range(L):
        lw = W["layers"][l]
        hs = [_norm(x, lw["attn_norm"], eps) for x in X]
        Q = [_mv(lw["wq"], h).reshape(H, hd) for h in hs]
        K = [_mv(lw["wk"], h).reshape(nkv, hd) for h in hs]
        V = [_mv(lw["wv"], h).reshape(nkv, hd) for h in hs]
        Q = [np.stack([_rotary(Q[p][a], p, cfg.rope_base) for a in range(H)]) for p in range(n)]
        K = [np.stack([_rotary(K[p][a], p, cfg.rope_base) for a in range(nkv)]) for p in range(n)]
        newX = []
        for i in range(n):
            outs = []
            for a in range(H):
                kv = a // G
                s = [float(np.dot(Q[i][a], K[j][kv])) / math.sqrt(hd) for j in range(i + 1)]
                m = max(s)
                e = [math.exp(v - m) for v in s]
                tot = sum(e)
                o = np.zeros(hd)
                for j in range(i + 1):
                    o += (e[j] / tot) * V[j][kv]
                outs.append(o)
            newX.append(X[i] + _mv(lw["wo"], np.concatenate(outs)))
        X = newX
        newX = []
        for i in range(n):
            h = _norm(X[i], lw["ffn_norm"], eps)
            if cfg.n_experts:
                r = _mv(lw["router"], h)
                m = max(r)
                e = [math.exp(v - m) for v in r]
                pr = [v / sum(e) for v in e]
                sel = sorted(range(cfg.n_experts), key=lambda k: (-pr[k], k))[:cfg.top_k]
                y = np.zeros_like(h)
                for s_ in range(cfg.n_shared_experts):
                    k = cfg.n_experts + s_
                    y += _swiglu(h, lw["e_gate"][k], lw["e_up"][k], lw["e_down"][k])
                tot = sum(pr[k] for k in sel) if getattr(cfg, "moe_renorm", False) else 1.0
                for k in sel:
                    y += (pr[k] / tot) * _swiglu(h, lw["e_gate"][k], lw["e_up"][k], lw["e_down"][k])
                if i == n - 1:
                    chosen.append(sel)
            else:
                y = _swiglu(h, lw["w_gate"], lw["w_up"], lw["w_down"])
            newX.append(X[i] + y)
        X = newX
    z = _mv(W["lm_head"], _norm(X[-1], W["final_norm"], eps))
    return (z, chosen) if return_experts else z
