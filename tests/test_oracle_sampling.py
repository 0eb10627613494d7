"""Pins of the oracle's temperature sampler (oracle/sampling.py) against
things other than itself: numpy's Philox4x64-10 bit generator, the Gumbel
distribution's closed-form mean, the softmax distribution the Gumbel-max
draw must follow, and its zero-temperature limit (the greedy argmax)."""
import numpy as np
import pytest

from oracle.decoder import argmax_first
from oracle.sampling import (MASK64, gumbel, philox4x64, philox4x64_vec, sample_keys, sample_token,
                             uniforms)


@pytest.mark.parametrize("key,ctr", [
    ((5, 7), (0, 0, 0, 0)),
    ((0, 0), (0, 0, 0, 0)),
    ((0xFFFFFFFFFFFFFFFF, 0x0123456789ABCDEF), (17, 3, 0, 9)),
    ((0x243F6A8885A308D3, 0x13198A2E03707344), (0xA4093822299F31D0, 0x082EFA98EC4E6C89, 1, 2)),
])
def test_philox_matches_numpy_bit_generator(key, ctr):
    # numpy's Philox bit generator is Philox4x64-10; it advances the counter
    # (word 0 first) before producing each 4-word block
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(ctr, dtype=np.uint64))
    raw = [int(x) for x in bg.random_raw(12)]
    for b in range(3):
        c = ((ctr[0] + 1 + b) & MASK64,) + tuple(ctr[1:])
        assert list(philox4x64(c, key)) == raw[4 * b: 4 * b + 4]


def test_vectorized_philox_matches_scalar():
    rng = np.random.default_rng(3)
    c = rng.integers(0, 2**63, size=(4, 64), dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    k0, k1 = 0x9E3779B97F4A7C15, 0x1234
    out = philox4x64_vec(c[0], c[1], c[2], c[3], k0, k1)
    for j in range(64):
        assert tuple(int(w[j]) for w in out) == philox4x64(tuple(int(x) for x in c[:, j]), (k0, k1))


def test_uniforms_lie_in_open_unit_interval_and_use_word_i_mod_4():
    u = uniforms(seed=11, pos=5, n=10)
    assert np.all(u > 0.0) and np.all(u < 1.0)
    # entry i is word i mod 4 of block i div 4 (counter (pos, i div 4, 0, 0), key (seed, 0))
    for i in range(10):
        w = philox4x64((5, i // 4, 0, 0), (11, 0))[i % 4]
        assert u[i] == ((w >> 11) + 0.5) * 2.0 ** -53


def test_gumbel_noise_has_the_closed_form_mean_and_variance():
    # Gumbel(0, 1): mean = Euler-Mascheroni gamma, variance = pi^2 / 6
    g = np.concatenate([gumbel(seed=7, pos=p, n=4096) for p in range(50)])   # 204,800 draws
    se = np.sqrt(np.pi ** 2 / 6 / g.size)
    assert abs(g.mean() - np.euler_gamma) < 5 * se
    assert abs(g.var() - np.pi ** 2 / 6) < 0.03


def test_gumbel_max_draws_follow_softmax_of_scaled_logits():
    z = np.array([0.3, -1.2, 0.9, 0.0, 2.1, -0.4, 1.5, 0.7], dtype=np.float32)
    t = 0.7
    n = 30000
    counts = np.bincount([sample_token(z, t, seed=123, pos=p) for p in range(n)], minlength=z.size)
    p = np.exp(z.astype(np.float64) / np.float32(t))
    p /= p.sum()
    expect = n * p
    chi2 = float(((counts - expect) ** 2 / expect).sum())
    # 7 degrees of freedom: P(chi2 > 30) ~ 1e-4
    assert chi2 < 30.0, (chi2, counts, expect)


def test_zero_temperature_limit_is_the_greedy_argmax():
    rng = np.random.default_rng(5)
    for pos in range(20):
        z = rng.standard_normal(512).astype(np.float32)
        assert sample_token(z, 1e-6, seed=9, pos=pos) == argmax_first(z)


def test_keys_depend_on_seed_and_position_only_through_the_noise():
    z = np.linspace(-1, 1, 64, dtype=np.float32)
    a = sample_keys(z, 1.0, seed=1, pos=0)
    assert np.array_equal(a, sample_keys(z, 1.0, seed=1, pos=0))
    assert not np.array_equal(a, sample_keys(z, 1.0, seed=2, pos=0))
    assert not np.array_equal(a, sample_keys(z, 1.0, seed=1, pos=1))


# ---- top-k / top-p
from oracle.sampling import MAX_TOP_K, candidate_order, kept_set, order_key, sample_token_topkp  # noqa: E402


def test_candidate_order_is_value_descending_then_index_ascending():
    z = np.array([1.0, 3.0, -2.0, 3.0, 0.0, -0.0, 1.0], dtype=np.float32)
    # by hand: 3.0 at 1 and 3, then 1.0 at 0 and 6, then +0.0 (4) above -0.0 (5), then -2.0
    assert list(candidate_order(z)) == [1, 3, 0, 6, 4, 5, 2]
    # the key order is the float order on a brute-force sweep of ordinary values
    rng = np.random.default_rng(0)
    v = rng.standard_normal(2000).astype(np.float32)
    k = order_key(v)
    i, j = rng.integers(0, 2000, size=(2, 5000))
    assert np.all((v[i] < v[j]) == (k[i] < k[j]))


def test_top_k_one_is_the_greedy_token_including_ties():
    rng = np.random.default_rng(1)
    for pos in range(40):
        z = np.round(rng.standard_normal(300), 1).astype(np.float32)   # many exact ties
        assert sample_token_topkp(z, 1.3, seed=77, pos=pos, top_k=1, top_p=1.0) == argmax_first(z)
    z = np.zeros(50, np.float32)
    assert sample_token_topkp(z, 1.0, seed=5, pos=3, top_k=1, top_p=1.0) == 0


def test_whole_vocabulary_pool_with_p_one_is_temperature_sampling():
    rng = np.random.default_rng(2)
    for pos in range(60):
        z = rng.standard_normal(200).astype(np.float32)
        want = sample_token(z, 0.9, seed=31, pos=pos)
        assert sample_token_topkp(z, 0.9, seed=31, pos=pos, top_k=200, top_p=1.0) == want
        assert sample_token_topkp(z, 0.9, seed=31, pos=pos, top_k=0, top_p=1.0) == want


def test_kept_sets_match_brute_force():
    rng = np.random.default_rng(3)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        z = np.round(rng.standard_normal(n) * 2, 1).astype(np.float32)
        t = float(rng.choice([0.3, 1.0, 2.5]))
        k = int(rng.integers(0, n + 3))
        p = float(rng.choice([1.0, 0.9, 0.5, 0.05]))
        keep = list(kept_set(z, t, k, p))
        # brute force: sort pairs (-value, index), take k (all if 0), then the
        # shortest prefix whose mass reaches p of the pool's mass
        pairs = sorted(range(n), key=lambda i: (-float(z[i]), i))
        pool = pairs[: min(k, n)] if k > 0 else pairs[: min(MAX_TOP_K, n)]
        if p < 1.0:
            q = [np.exp((float(z[i]) - float(z[pool[0]])) / float(np.float32(t))) for i in pool]
            tot = float(np.cumsum(q)[-1])
            run, m = 0.0, 0
            for m, qi in enumerate(q, 1):
                run += qi
                if run >= float(np.float32(p)) * tot:
                    break
            pool = pool[:m]
        assert keep == pool, (z, t, k, p, keep, pool)


def _chi2(counts, probs, n):
    expect = n * probs
    return float(((counts - expect) ** 2 / expect).sum())


def test_top_k_draws_follow_the_renormalised_softmax():
    z = np.array([0.3, -1.2, 0.9, 0.0, 2.1, -0.4, 1.5, 0.7, -2.0, 0.1], dtype=np.float32)
    t, k, n = 0.8, 4, 30000
    draws = [sample_token_topkp(z, t, seed=99, pos=p, top_k=k, top_p=1.0) for p in range(n)]
    counts = np.bincount(draws, minlength=z.size)
    top = np.argsort(-z.astype(np.float64), kind="stable")[:k]
    assert set(np.nonzero(counts)[0]) <= set(top.tolist())
    q = np.exp(z[top].astype(np.float64) / np.float32(t))
    # 3 degrees of freedom: P(chi2 > 21) ~ 1e-4
    assert _chi2(counts[top], q / q.sum(), n) < 21.0


def test_top_p_draws_follow_the_renormalised_nucleus():
    z = np.array([2.0, 1.6, 1.0, 0.2, -0.5, -1.0, 0.9, 1.7], dtype=np.float32)
    t, p, n = 1.0, 0.8, 30000
    # nucleus by hand: probabilities sorted 2.0, 1.7, 1.6, 1.0, 0.9, 0.2, -0.5, -1.0
    w = np.exp(np.array([2.0, 1.7, 1.6, 1.0, 0.9, 0.2, -0.5, -1.0]))
    cum = np.cumsum(w) / w.sum()
    m = int(np.argmax(cum >= np.float32(p))) + 1
    assert m == 4                                                       # cum 0.29, 0.51, 0.71, 0.82
    want = [0, 7, 1, 2]
    assert list(kept_set(z, t, 0, p)) == want
    draws = [sample_token_topkp(z, t, seed=4, pos=i, top_k=0, top_p=p) for i in range(n)]
    counts = np.bincount(draws, minlength=z.size)
    assert set(np.nonzero(counts)[0]) <= set(want)
    q = np.exp(z[want].astype(np.float64))
    assert _chi2(counts[want], q / q.sum(), n) < 25.0                  # m - 1 degrees of freedom
