"""Plain numpy decoder: the definition the persistent decode kernel must reproduce.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path imports this module.

Source of each step
-------------------
* Decode at batch 1 streams every active weight once per generated token and
  is bound by memory bandwidth (page "Breaking the memory wall: 3,000 tokens/s
  inference on standard GPUs", section "The bottleneck: memory bandwidth, not
  compute"); that is why the weights stay fp16 in memory here too and are
  only widened for the arithmetic.
* The path consists of matrix multiplies, attention, normalisation and
  sampling (same page, section "1. The Monokernel Runtime").
* Only active parameters are moved for a mixture-of-experts model (same page,
  section "Scaling to frontier MoE models"): :func:`moe_ffn` touches only the
  selected experts.

The layer structure itself is not on the pages.  The workloads name its parts
(RMSNorm eps 1e-5, RoPE base 10000, SwiGLU FFN, MHA/GQA, untied embeddings,
greedy decoding, softmax top-k routing plus shared experts); the plain
pre-norm reading is used:  x += Attn(rms(x)); x += FFN(rms(x)); logits =
lm_head(rms(x)).  Linears are bias-free and row-major ``[out][in]``.
"""
from __future__ import annotations

from collections import OrderedDict
from typing import Optional, Sequence

import numpy as np


# ----------------------------------------------------------------------------
# Building blocks (each is written as the textbook definition)
# ----------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gain.

    eps sits inside the square root (plain reading; the workload only gives
    its value, 1e-5)."""
    dt = x.dtype
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return (x / np.sqrt(ms + dt.type(eps))) * gain.astype(dt)


def rope_cos_sin(positions, head_dim: int, base: float, dtype=np.float32):
    """Rotary angles: theta_j = base^(-2j/head_dim), j < head_dim/2, angle p*theta_j.

    Angles and their cos/sin are formed in float64 and rounded once to
    ``dtype``.  Returns arrays of shape ``positions.shape + (head_dim/2,)``."""
    half = head_dim // 2
    j = np.arange(half, dtype=np.float64)
    theta = np.power(np.float64(base), -2.0 * j / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[..., None] * theta
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope(v: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE: element j pairs with element j + head_dim/2.

    v'[j] = v[j] c_j - v[j+h] s_j ;  v'[j+h] = v[j+h] c_j + v[j] s_j.
    (The pairing is this code's reading; the workload names RoPE and its
    base only.)"""
    half = v.shape[-1] // 2
    a = v[..., :half]
    b = v[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    """exp(s - max s) / sum(exp(s - max s)) along ``axis``."""
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """One query against keys/values 0..n-1: softmax(K q / sqrt(hd)) V.

    Causal masking is the caller's slice (all positions up to and including
    the query's own)."""
    dt = q.dtype
    scale = dt.type(1.0 / np.sqrt(np.float64(q.shape[-1])))
    s = (K @ q) * scale
    return softmax(s) @ V


def silu(a: np.ndarray) -> np.ndarray:
    """SiLU (swish-1): a * sigmoid(a) = a / (1 + exp(-a))."""
    one = a.dtype.type(1.0)
    return a / (one + np.exp(-a))


def swiglu(h: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """SwiGLU FFN: W_down (silu(W_gate h) * (W_up h)).  Works on [d] or [n, d]."""
    if h.ndim == 1:
        return w_down @ (silu(w_gate @ h) * (w_up @ h))
    return (silu(h @ w_gate.T) * (h @ w_up.T)) @ w_down.T


def argmax_first(z: np.ndarray) -> int:
    """Greedy token: index of the largest logit, the lowest index on ties."""
    return int(np.argmax(z))     # numpy returns the first maximal index


def moe_route(r: np.ndarray, top_k: int):
    """Softmax over all router logits, then the ``top_k`` largest probabilities.

    Ties go to the lower expert index (stable order).  The selected
    probabilities are used as mixing weights as they are, not renormalised:
    the workload says "softmax top-k", and softmax-then-select is its plain
    reading.  Returns (probabilities, selected expert ids in rank order)."""
    pi = softmax(r)
    order = np.argsort(-pi, kind="stable")
    return pi, order[:top_k]


def moe_ffn(h: np.ndarray, router: np.ndarray, expert, n_experts: int, top_k: int,
            n_shared: int, router_log: Optional[list] = None, renorm: bool = False) -> tuple:
    """Mixture-of-experts FFN for one token.

    y = sum over shared experts s of SwiGLU_s(h) + sum over the selected routed
    experts e of w_e * SwiGLU_e(h), with w_e = pi_e, or, with ``renorm`` (the
    other common reading of "softmax top-k"), w_e = pi_e / (sum of pi over the
    selected experts), so that the routed weights sum to 1.  ``expert(e)`` returns the widened
    (gate, up, down) of expert e; ids n_experts.. are the shared experts.
    Only the experts used are touched (active-parameter streaming).
    Returns (y, selected ids); the router logits are appended to
    ``router_log`` when one is given (for judging near-ties in routing)."""
    r = router @ h
    if router_log is not None:
        router_log.append(r)
    pi, sel = moe_route(r, top_k)
    w = pi / pi[sel].sum() if renorm else pi
    y = np.zeros_like(h)
    for s in range(n_shared):
        g, u, d = expert(n_experts + s)
        y = y + swiglu(h, g, u, d)
    for e in sel:
        g, u, d = expert(int(e))
        y = y + w[e] * swiglu(h, g, u, d)
    return y, sel


# ----------------------------------------------------------------------------
# The decoder
# ----------------------------------------------------------------------------

class Oracle:
    """Batch-1 decoder over fp16 weights, computing in ``dtype`` (fp32 default).

    State: the KV cache (kept in ``dtype``; ``kv_fp16=True`` rounds stored rows
    to fp16, a diagnosis switch only), the next position ``pos`` and the
    pending token.

    Prefill/decode convention (the pages name neither call's semantics; this
    is the reading that makes every logit vector a decode output):
    ``prefill(t)`` runs positions 0..P-2 and leaves ``t[P-1]`` pending at
    ``pos = P-1``; decode step i runs the model on the pending token at
    position P-1+i, emits its logits and greedy token g_i, and g_i (or
    ``force[i]``) becomes pending.
    """

    def __init__(self, cfg, weights: dict, dtype=np.float32, kv_fp16: bool = False,
                 cache_bytes: int = 1 << 62):
        self.cfg = cfg
        self.w = weights
        self.dt = np.dtype(dtype)
        self.kv_fp16 = kv_fp16
        self._cache: "OrderedDict[tuple, np.ndarray]" = OrderedDict()
        self._cache_bytes = 0
        self._cache_limit = cache_bytes
        self.expert_log = []        # per decode step: [layer] -> selected ids
        self.router_log = []        # per decode step: [layer] -> router logits
        self.route = {}             # position -> (ids [L][top_k], router logits [L][E])
        self.reset()

    # -- weights ----------------------------------------------------------
    def _wide(self, key: tuple, fetch) -> np.ndarray:
        """fp16 -> dtype widening, cached (exact: every fp16 is an fp32)."""
        a = self._cache.get(key)
        if a is not None:
            self._cache.move_to_end(key)
            return a
        a = np.ascontiguousarray(fetch(), dtype=self.dt)
        self._cache[key] = a
        self._cache_bytes += a.nbytes
        while self._cache_bytes > self._cache_limit and len(self._cache) > 1:
            _, old = self._cache.popitem(last=False)
            self._cache_bytes -= old.nbytes
        return a

    def lw(self, l: int, name: str) -> np.ndarray:
        return self._wide((l, name), lambda: self.w["layers"][l][name])

    def gw(self, name: str) -> np.ndarray:
        return self._wide(("g", name), lambda: self.w[name])

    def expert(self, l: int, e: int):
        lw = self.w["layers"][l]
        return (self._wide((l, "e_gate", e), lambda: lw["e_gate"][e]),
                self._wide((l, "e_up", e), lambda: lw["e_up"][e]),
                self._wide((l, "e_down", e), lambda: lw["e_down"][e]))

    # -- state ------------------------------------------------------------
    def reset(self):
        c = self.cfg
        cap = c.kv_capacity
        self.K = [np.zeros((c.n_kv_heads, cap, c.head_dim), self.dt) for _ in range(c.n_layers)]
        self.V = [np.zeros((c.n_kv_heads, cap, c.head_dim), self.dt) for _ in range(c.n_layers)]
        self.pos = 0
        self.pending: Optional[int] = None
        self.expert_log = []
        self.router_log = []
        self.route = {}

    def _store_kv(self, l, p, k, v):
        if self.kv_fp16:
            k = k.astype(np.float16).astype(self.dt)
            v = v.astype(np.float16).astype(self.dt)
        self.K[l][:, p] = k
        self.V[l][:, p] = v

    def _ffn(self, l: int, h: np.ndarray, router_log: Optional[list] = None):
        c = self.cfg
        if not c.is_moe:
            return swiglu(h, self.lw(l, "w_gate"), self.lw(l, "w_up"), self.lw(l, "w_down")), None
        return moe_ffn(h, self.lw(l, "router"), lambda e: self.expert(l, e),
                       c.n_experts, c.top_k, c.n_shared_experts, router_log,
                       renorm=getattr(c, "moe_renorm", False))

    # -- one token ----------------------------------------------------------
    def step(self, tok: int) -> np.ndarray:
        """Run the model on ``tok`` at position ``self.pos``; returns logits [vocab_out]."""
        c = self.cfg
        p = self.pos
        if p >= c.kv_capacity:
            raise ValueError("context overflow")
        if not 0 <= tok < c.vocab_in:
            raise ValueError("token id out of range")
        H, G, hd = c.n_heads, c.n_heads // c.n_kv_heads, c.head_dim
        eps = c.rms_eps
        x = self.w["tok_emb"][tok].astype(self.dt)
        cos, sin = rope_cos_sin(p, hd, c.rope_base, self.dt)
        experts, router = [], []
        for l in range(c.n_layers):
            h = rmsnorm(x, self.w["layers"][l]["attn_norm"], eps)
            q = (self.lw(l, "wq") @ h).reshape(H, hd)
            k = (self.lw(l, "wk") @ h).reshape(c.n_kv_heads, hd)
            v = (self.lw(l, "wv") @ h).reshape(c.n_kv_heads, hd)
            q = rope(q, cos, sin)
            k = rope(k, cos, sin)
            self._store_kv(l, p, k, v)
            o = np.empty((H, hd), self.dt)
            for i in range(H):
                g = i // G                      # query head i reads KV head i // G
                o[i] = attend(q[i], self.K[l][g, :p + 1], self.V[l][g, :p + 1])
            x = x + self.lw(l, "wo") @ o.reshape(-1)
            h = rmsnorm(x, self.w["layers"][l]["ffn_norm"], eps)
            y, sel = self._ffn(l, h, router)
            if sel is not None:
                experts.append(np.asarray(sel, np.int32))
            x = x + y
        self.pos = p + 1
        if experts:
            self.expert_log.append(np.stack(experts))
            self.router_log.append(np.stack(router))
            self.route[p] = (self.expert_log[-1], self.router_log[-1])
        return self.gw("lm_head") @ rmsnorm(x, self.w["final_norm"], eps)

    # -- prompt ---------------------------------------------------------------
    def prefill(self, tokens: Sequence[int], batched: bool = True):
        """Fill the KV cache for positions 0..P-2 and leave tokens[P-1] pending."""
        c = self.cfg
        t = np.asarray(tokens, dtype=np.int64)
        P = len(t)
        if self.pos != 0 or self.pending is not None:
            raise ValueError("prefill needs a fresh state")
        if P < 1 or P > c.kv_capacity:
            raise ValueError("bad prompt length")
        if np.any(t < 0) or np.any(t >= c.vocab_in):
            raise ValueError("token id out of range")
        if P > 1:
            if batched:
                self._prefill_batched(t[:-1])
            else:
                for tok in t[:-1]:
                    self.step(int(tok))
            self.expert_log = []
            self.router_log = []
        self.pos = P - 1
        self.pending = int(t[-1])

    def _prefill_batched(self, t: np.ndarray):
        """All prompt positions at once: the same arithmetic with a causal mask."""
        c = self.cfg
        n = len(t)
        H, G, hd = c.n_heads, c.n_heads // c.n_kv_heads, c.head_dim
        eps = c.rms_eps
        X = self.w["tok_emb"][t].astype(self.dt)                      # [n, d]
        cos, sin = rope_cos_sin(np.arange(n), hd, c.rope_base, self.dt)
        cos, sin = cos[:, None, :], sin[:, None, :]                    # [n, 1, half]
        scale = self.dt.type(1.0 / np.sqrt(np.float64(hd)))
        future = np.triu(np.ones((n, n), dtype=bool), k=1)             # key j > query i
        for l in range(c.n_layers):
            Hn = rmsnorm(X, self.w["layers"][l]["attn_norm"], eps)
            Q = rope((Hn @ self.lw(l, "wq").T).reshape(n, H, hd), cos, sin)
            Kx = rope((Hn @ self.lw(l, "wk").T).reshape(n, c.n_kv_heads, hd), cos, sin)
            Vx = (Hn @ self.lw(l, "wv").T).reshape(n, c.n_kv_heads, hd)
            for p in range(n):
                self._store_kv(l, p, Kx[p], Vx[p])
            O = np.empty((n, H, hd), self.dt)
            for i in range(H):
                g = i // G
                Kc, Vc = self.K[l][g, :n], self.V[l][g, :n]
                S = (Q[:, i, :] @ Kc.T) * scale                         # [n, n]
                S[future] = -np.inf
                O[:, i, :] = softmax(S, axis=-1) @ Vc
            X = X + O.reshape(n, H * hd) @ self.lw(l, "wo").T
            Hn = rmsnorm(X, self.w["layers"][l]["ffn_norm"], eps)
            if c.is_moe:
                Y = self._moe_prompt(l, Hn)
            else:
                Y = swiglu(Hn, self.lw(l, "w_gate"), self.lw(l, "w_up"), self.lw(l, "w_down"))
            X = X + Y
        for p in list(self.route):
            ids, rl = self.route[p]
            self.route[p] = (np.stack(ids), np.stack(rl))

    def _moe_prompt(self, l: int, Hn: np.ndarray) -> np.ndarray:
        """The mixture-of-experts FFN of layer ``l`` for every prompt position.

        Each position is routed exactly as :func:`moe_ffn` routes one token
        (its own router matrix-vector product, softmax, top-k).  Each expert's
        SwiGLU is then applied to all the positions that use it as one matrix
        product (the same formula, row by row), and position p sums its
        experts in :func:`moe_ffn`'s order: shared experts, then the routed
        ones by rank.  Appends the routing to ``self.route``."""
        c = self.cfg
        n = Hn.shape[0]
        E, S = c.n_experts, c.n_shared_experts
        renorm = getattr(c, "moe_renorm", False)
        router = self.lw(l, "router")
        sel_all, w_all = [], []
        users = [[] for _ in range(E + S)]
        for p in range(n):
            r = router @ Hn[p]
            pi, sel = moe_route(r, c.top_k)
            w = pi / pi[sel].sum() if renorm else pi
            sel_all.append(sel)
            w_all.append(w)
            for e in sel:
                users[int(e)].append(p)
            ids, rl = self.route.get(p, ([], []))
            self.route[p] = (list(ids) + [np.asarray(sel, np.int32)], list(rl) + [r])
        for s in range(S):
            users[E + s] = list(range(n))
        out = [None] * (E + S)                # expert e -> {position: SwiGLU_e(h_p)}
        for e in range(E + S):
            if users[e]:
                g, u, d = self.expert(l, e)
                rows = np.asarray(users[e])
                out[e] = dict(zip(users[e], swiglu(Hn[rows], g, u, d)))
        Y = np.zeros_like(Hn)
        for p in range(n):
            y = Y[p]
            for s in range(S):
                y = y + out[E + s][p]
            for e in sel_all[p]:
                y = y + w_all[p][e] * out[int(e)][p]
            Y[p] = y
        return Y

    # -- generation -------------------------------------------------------------
    def decode(self, n: int, force: Optional[Sequence[int]] = None, keep_logits: bool = True):
        """n greedy steps.  With ``force``, step i's output token is still the
        oracle's own argmax, but ``force[i]`` becomes the next input
        (teacher forcing onto another decoder's tokens).  Returns
        (tokens int32 [n], logits [n, vocab_out] or None)."""
        if self.pending is None:
            raise ValueError("decode needs a pending token (call prefill)")
        c = self.cfg
        if self.pos + n > c.kv_capacity:
            raise ValueError("context overflow")
        toks = np.empty(n, np.int32)
        logits = np.empty((n, c.vocab_out), self.dt) if keep_logits else None
        for i in range(n):
            z = self.step(self.pending)
            toks[i] = argmax_first(z)
            if keep_logits:
                logits[i] = z
            self.pending = int(force[i]) if force is not None else int(toks[i])
        return toks, logits
