"""The pins must catch plausible oracle mistakes.  Each case plants one mistake
in the oracle (monkeypatched, CPU only) and checks that the brute-force
comparison then fails."""
import numpy as np
import pytest

import oracle.decoder as dec
from kie_synth import make_prompt, make_weights, weights_to_numpy
from tests import brute
from tests.test_oracle_pins import SMALL_GQA, SMALL_MOE

_orig_rope, _orig_attend, _orig_rms, _orig_silu, _orig_route = (
    dec.rope, dec.attend, dec.rmsnorm, dec.silu, dec.moe_route)


def _rope_sign(v, c, s):
    h = v.shape[-1] // 2
    a, b = v[..., :h], v[..., h:]
    return np.concatenate([a * c + b * s, b * c - a * s], axis=-1)


def _rope_interleaved(v, c, s):
    a, b = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = b * c + a * s
    return out


def _attend_noscale(q, K, V):
    return dec.softmax(K @ q) @ V


def _rms_eps_outside(x, g, eps):
    return (x / (np.sqrt(np.mean(x * x, -1, keepdims=True)) + x.dtype.type(eps))) * g.astype(x.dtype)


def _silu_as_sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def _route_renorm(r, k):
    pi, sel = _orig_route(r, k)
    pi = pi.copy()
    pi[sel] = pi[sel] / pi[sel].sum()
    return pi, sel


MUTANTS = {
    "rope_sign": ("rope", _rope_sign),
    "rope_interleaved": ("rope", _rope_interleaved),
    "attention_scale_dropped": ("attend", _attend_noscale),
    "rms_eps_outside_sqrt": ("rmsnorm", _rms_eps_outside),
    "silu_dropped_factor": ("silu", _silu_as_sigmoid),
    "moe_renormalised": ("moe_route", _route_renorm),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(monkeypatch, name):
    attr, fn = MUTANTS[name]
    cfg = SMALL_MOE if name.startswith("moe") else SMALL_GQA
    W = weights_to_numpy(make_weights(cfg, seed=3, std=0.3))
    prompt = make_prompt(cfg, seed=1)
    monkeypatch.setattr(dec, attr, fn)
    o = dec.Oracle(cfg, W, dtype=np.float64)
    o.prefill(prompt)
    _, z = o.decode(2)
    want = brute.last_logits(cfg, W, list(prompt))
    assert not np.allclose(z[0], want, rtol=1e-6, atol=1e-8), name


def test_planted_gqa_index_mistake_is_caught(monkeypatch):
    # query head i must read KV head i // G, not i % n_kv
    cfg = SMALL_GQA
    W = weights_to_numpy(make_weights(cfg, seed=3, std=0.3))
    prompt = make_prompt(cfg, seed=1)

    class Wrong(dec.Oracle):
        def step(self, tok):
            c = self.cfg
            p = self.pos
            H, hd = c.n_heads, c.head_dim
            x = self.w["tok_emb"][tok].astype(self.dt)
            cos, sin = dec.rope_cos_sin(p, hd, c.rope_base, self.dt)
            for l in range(c.n_layers):
                h = dec.rmsnorm(x, self.w["layers"][l]["attn_norm"], c.rms_eps)
                q = dec.rope((self.lw(l, "wq") @ h).reshape(H, hd), cos, sin)
                k = dec.rope((self.lw(l, "wk") @ h).reshape(c.n_kv_heads, hd), cos, sin)
                v = (self.lw(l, "wv") @ h).reshape(c.n_kv_heads, hd)
                self._store_kv(l, p, k, v)
                o = np.stack([dec.attend(q[i], self.K[l][i % c.n_kv_heads, :p + 1],
                                         self.V[l][i % c.n_kv_heads, :p + 1]) for i in range(H)])
                x = x + self.lw(l, "wo") @ o.reshape(-1)
                x = x + self._ffn(l, dec.rmsnorm(x, self.w["layers"][l]["ffn_norm"], c.rms_eps))[0]
            self.pos = p + 1
            return self.gw("lm_head") @ dec.rmsnorm(x, self.w["final_norm"], c.rms_eps)

    o = Wrong(cfg, W, dtype=np.float64)
    o.prefill(prompt, batched=False)
    _, z = o.decode(1)
    want = brute.last_logits(cfg, W, list(prompt))
    assert not np.allclose(z[0], want, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("name", ["wq", "wo"])
def test_planted_transposed_operand_is_caught(name):
    # a square projection (d_model == n_heads * head_dim in the small
    # workload) applied transposed still runs, so only the pins can catch it
    cfg = SMALL_GQA
    W = weights_to_numpy(make_weights(cfg, seed=3, std=0.3))
    prompt = make_prompt(cfg, seed=1)
    assert W["layers"][0][name].shape[0] == W["layers"][0][name].shape[1]

    class Transposed(dec.Oracle):
        def lw(self, l, nm):
            w = super().lw(l, nm)
            return w.T if nm == name else w

    o = Transposed(cfg, W, dtype=np.float64)
    o.prefill(prompt)
    _, z = o.decode(1)
    want = brute.last_logits(cfg, W, list(prompt))
    assert not np.allclose(z[0], want, rtol=1e-6, atol=1e-8), name
