"""Stochastic sampling for the oracle — TEST INFRASTRUCTURE (see the package
docstring: only tests/, the smoke check and the bench's CPU-baseline leg may
use it).

The pages put sampling inside the monokernel (page "Breaking the memory wall:
3,000 tokens/s inference on standard GPUs", agentlenshq.com, section "1. The
Monokernel Runtime": the one GPU-resident program does the matrix multiplies,
attention, normalisation and sampling).  They name no sampling rule; the
plainest exact reading is temperature sampling, a draw from softmax(z / T),
and this module defines it the way the decode kernel computes it:

* Random numbers come from Philox4x64-10, the counter-based generator of
  Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3"
  (SC 2011): ten rounds of two 64x64->128-bit multiplies with the key bumped
  by two Weyl constants between rounds.  Vocabulary entry i of the decode step
  at position `pos` with seed `seed` uses word (i mod 4) of the block for
  counter (pos, i div 4, 0, 0) and key (seed, 0).
* The draw is the Gumbel-max method: with u_i uniform in (0, 1) and
  g_i = -log(-log(u_i)), argmax_i (z_i / T + g_i) is distributed as
  softmax(z / T) (Gumbel 1954; the "Gumbel-max trick").  u_i is the top 53
  bits of the Philox word, centred in its bin: ((w >> 11) + 0.5) * 2^-53, so
  it is never 0 or 1.
* The keys z_i / T + g_i are formed in float64 from the float32 logits and
  the float32 temperature, rounded once to float32, and the first maximum
  wins (the kernel folds packed float32 keys into the same argmax it uses for
  greedy decoding).

Top-k and top-p (nucleus) sampling restrict that draw to a candidate set
and are not defined on the pages either; the reading taken here:

* Candidates are ordered by logit, largest first, ties by the lower index
  (exactly the order of the greedy argmax).  Top-k keeps the first k of
  them; with top-p and no top-k the pool is the first MAX_TOP_K (256), so a
  nucleus wider than that is cut there.
* Top-p then keeps the shortest prefix of the pool whose probability mass
  reaches p times the pool's mass: q_j = exp((z_j - z_0) / T) in float64
  (z_0 the largest logit), c = the running sum of q in pool order, and the
  prefix ends at the first j with c_j >= p * c_last.
* The token is the Gumbel-max draw (the keys above) over the kept set, the
  first maximum (lowest index) winning.  Top-k 1 is therefore the greedy
  token, and a pool of the whole vocabulary with p = 1 is plain temperature
  sampling.

Parity status: Philox is pinned against numpy's own Philox4x64-10 bit
generator; the draw against the softmax distribution (chi-square over many
counters), its zero-temperature limit (the greedy argmax) and its shift
invariance; top-k 1 against the greedy argmax, the whole-vocabulary pool
against temperature sampling, the kept sets against brute force and the
draws against the renormalised truncated softmax (chi-square).  See
tests/test_oracle_sampling.py.
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
# Philox4x64 multipliers and Weyl key increments (Salmon et al. 2011)
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B
PHILOX_ROUNDS = 10


def philox4x64(ctr, key, rounds: int = PHILOX_ROUNDS):
    """One Philox4x64 block, exact, on Python integers.

    ctr: four 64-bit words, key: two 64-bit words.  Each round multiplies
    words 0 and 2 by the two multipliers (128-bit products split into high
    and low halves) and mixes: (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the
    key is bumped by the Weyl constants after every round."""
    c0, c1, c2, c3 = (int(x) & MASK64 for x in ctr)
    k0, k1 = (int(x) & MASK64 for x in key)
    for _ in range(rounds):
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        hi0, lo0 = p0 >> 64, p0 & MASK64
        hi1, lo1 = p1 >> 64, p1 & MASK64
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        k0 = (k0 + PHILOX_W0) & MASK64
        k1 = (k1 + PHILOX_W1) & MASK64
    return c0, c1, c2, c3


_M32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo64(a: np.ndarray, m: int):
    """128-bit product of uint64 array `a` and constant `m`: (high, low),
    through 32-bit limbs so every partial product fits in 64 bits."""
    a_lo, a_hi = a & _M32, a >> _S32
    m_lo, m_hi = np.uint64(m & 0xFFFFFFFF), np.uint64(m >> 32)
    ll = a_lo * m_lo
    hl = a_hi * m_lo
    lh = a_lo * m_hi
    hh = a_hi * m_hi
    mid = (ll >> _S32) + (hl & _M32) + (lh & _M32)
    hi = hh + (hl >> _S32) + (lh >> _S32) + (mid >> _S32)
    lo = (mid << _S32) | (ll & _M32)
    return hi, lo


def philox4x64_vec(c0, c1, c2, c3, k0: int, k1: int, rounds: int = PHILOX_ROUNDS):
    """philox4x64 over arrays of counters (uint64), same key for all."""
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64).copy() for x in (c0, c1, c2, c3))
    with np.errstate(over="ignore"):
        for r in range(rounds):
            kk0 = np.uint64((k0 + r * PHILOX_W0) & MASK64)
            kk1 = np.uint64((k1 + r * PHILOX_W1) & MASK64)
            hi0, lo0 = _mulhilo64(c0, PHILOX_M0)
            hi1, lo1 = _mulhilo64(c2, PHILOX_M1)
            c0, c1, c2, c3 = hi1 ^ c1 ^ kk0, lo1, hi0 ^ c3 ^ kk1, lo0
    return c0, c1, c2, c3


def uniforms(seed: int, pos: int, n: int) -> np.ndarray:
    """u_i in (0, 1), float64, for vocabulary entries 0..n-1 at `pos`."""
    blocks = (n + 3) // 4
    j = np.arange(blocks, dtype=np.uint64)
    zero = np.zeros(blocks, dtype=np.uint64)
    out = philox4x64_vec(np.full(blocks, pos & MASK64, dtype=np.uint64), j, zero, zero,
                         int(seed) & MASK64, 0)
    words = np.stack(out, axis=1).reshape(-1)[:n]          # entry i: word i mod 4 of block i div 4
    return ((words >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53


def gumbel(seed: int, pos: int, n: int) -> np.ndarray:
    """Gumbel(0, 1) noise g_i = -log(-log(u_i)), float64."""
    return -np.log(-np.log(uniforms(seed, pos, n)))


def sample_keys(z: np.ndarray, temperature: float, seed: int, pos: int) -> np.ndarray:
    """float32 keys z_i / T + g_i (formed in float64, rounded once)."""
    z64 = np.asarray(z, dtype=np.float32).astype(np.float64)
    t = float(np.float32(temperature))
    return (z64 / t + gumbel(seed, pos, z64.shape[0])).astype(np.float32)


def sample_token(z: np.ndarray, temperature: float, seed: int, pos: int) -> int:
    """One draw from softmax(z / T): the first maximum of the keys."""
    keys = sample_keys(z, temperature, seed, pos)
    return int(np.argmax(keys))


MAX_TOP_K = 256        # candidate pool of top-k / top-p sampling, at most


def order_key(z: np.ndarray) -> np.ndarray:
    """uint32 keys whose unsigned order is the float32 order of z (-0 below +0)."""
    u = np.asarray(z, dtype=np.float32).view(np.uint32).astype(np.uint64)
    neg = (u & np.uint64(0x80000000)) != 0
    return np.where(neg, np.uint64(0xFFFFFFFF) - u, u | np.uint64(0x80000000)).astype(np.uint64)


def candidate_order(z: np.ndarray) -> np.ndarray:
    """Vocabulary indices by logit, largest first, ties by the lower index."""
    k = order_key(z)
    idx = np.arange(k.shape[0])
    return np.lexsort((idx, -k.astype(np.int64)))


def kept_set(z: np.ndarray, temperature: float, top_k: int, top_p: float) -> np.ndarray:
    """Indices (in candidate order) that top-k then top-p keep."""
    V = int(np.asarray(z).shape[0])
    K = min(top_k if top_k > 0 else MAX_TOP_K, V)
    pool = candidate_order(z)[:K]
    if top_p < 1.0:
        z64 = np.asarray(z, dtype=np.float32).astype(np.float64)
        t = float(np.float32(temperature))
        q = np.exp((z64[pool] - z64[pool[0]]) / t)
        c = np.cumsum(q)
        m = int(np.argmax(c >= float(np.float32(top_p)) * c[-1])) + 1
        pool = pool[:m]
    return pool


def sample_token_topkp(z: np.ndarray, temperature: float, seed: int, pos: int, top_k: int,
                       top_p: float) -> int:
    """One draw restricted by top-k (0: none) and top-p (1: none)."""
    if top_k == 0 and top_p >= 1.0:
        return sample_token(z, temperature, seed, pos)
    keep = kept_set(z, temperature, top_k, top_p)
    keys = sample_keys(z, temperature, seed, pos)[keep]
    best = keys.max()
    return int(keep[keys == best].min())
