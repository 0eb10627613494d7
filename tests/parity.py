"""Teacher-forced comparison of GPU decode output with the oracle.

Tolerances (the workload's stated bar): per step, max |z_gpu - z_oracle| is
at most 2e-2 and at most 1e-2 of the oracle's logit range for that step;
the greedy token must equal the oracle's argmax wherever the oracle's
top-2 margin exceeds 5e-2; token ids and positions are exact.
"""
from __future__ import annotations

import numpy as np

ABS_TOL = 2e-2
REL_RANGE_TOL = 1e-2
MARGIN = 5e-2


def compare_steps(z_gpu: np.ndarray, tok_gpu: np.ndarray, z_or: np.ndarray, skip=()):
    """Returns a report dict; raises AssertionError on the first failing step.

    Every step, pinned or not, is held to these checks:
    - the logit bar (absolute, and relative to the oracle's range);
    - the token is the first maximum of the kernel's own logits.  This is
      exact: the kernel takes its argmax over the same float32 values it
      writes out, lowest index on ties.  It checks the on-device argmax and
      the feedback of its token into the next step;
    - the token is a valid greedy choice for the oracle: if every logit is
      within e of the oracle's, then the chosen logit is within 2e of the
      oracle's maximum.  Where the oracle's third logit is more than 2e below
      its maximum, this means the token is one of the oracle's top two.
    Steps whose oracle top-2 margin exceeds ``MARGIN`` must match the
    oracle's argmax exactly ("pinned")."""
    n = len(tok_gpu)
    pinned = unpinned = 0
    worst = 0.0
    for i in range(n):
        if i in skip:
            continue
        zo = z_or[i].astype(np.float64)
        zg = z_gpu[i].astype(np.float64)
        tok = int(tok_gpu[i])
        err = float(np.max(np.abs(zg - zo)))
        rng = float(zo.max() - zo.min())
        worst = max(worst, err)
        assert err <= ABS_TOL, f"step {i}: max |dz| = {err:.3e} > {ABS_TOL}"
        assert err <= REL_RANGE_TOL * rng, f"step {i}: max |dz| = {err:.3e} > 1e-2 * range {rng:.3f}"
        assert tok == int(np.argmax(z_gpu[i])), (
            f"step {i}: gpu token {tok} is not the first maximum {int(np.argmax(z_gpu[i]))} "
            f"of the gpu's own logits")
        zmax = float(zo.max())
        assert zo[tok] >= zmax - 2.0 * ABS_TOL, (
            f"step {i}: gpu token {tok} has oracle logit {zo[tok]:.4f}, more than "
            f"{2 * ABS_TOL} below the oracle maximum {zmax:.4f}")
        top3 = np.sort(np.partition(zo, -3)[-3:])
        if top3[0] < zmax - 2.0 * ABS_TOL:
            top2_ids = np.argsort(-zo, kind="stable")[:2]
            assert tok in top2_ids, f"step {i}: gpu token {tok} not in oracle top-2 {top2_ids.tolist()}"
        margin = float(top3[2] - top3[1])
        if margin > MARGIN:
            pinned += 1
            assert tok == int(np.argmax(zo)), (
                f"step {i}: gpu token {tok} != oracle argmax {int(np.argmax(zo))} "
                f"(margin {margin:.3f})")
        else:
            unpinned += 1
    return {"steps": n, "pinned": pinned, "unpinned": unpinned, "worst_abs": worst}


def _fp16_ulp(a: np.ndarray) -> np.ndarray:
    """Spacing of fp16 numbers at |a| (2^-24 in the subnormal range)."""
    a = np.abs(a).astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def kv_close(k_gpu_f16: np.ndarray, k_or: np.ndarray, what: str, ulps: float = 0.5,
             rel: float = 1e-5):
    """fp16 cache rows of the first layer against the oracle's fp32 rows.

    The first layer's K/V rows depend only on the token at that position,
    so both sides start from identical inputs; the only differences are the
    fp16 rounding of the stored row (half an fp16 ulp) and fp32 summation
    order (``rel``)."""
    g = k_gpu_f16.astype(np.float64)
    o = k_or.astype(np.float64)
    tol = ulps * _fp16_ulp(o) + rel * np.maximum(1.0, np.abs(o))
    bad = np.abs(g - o) > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} KV elements off, worst "
                           f"{float(np.max(np.abs(g - o))):.3e}")


KV_ROW_REL = 6e-3


def kv_rows_close(k_gpu_f16: np.ndarray, k_or: np.ndarray, what: str, rel: float = KV_ROW_REL):
    """Cache rows of any layer against the oracle's fp32 rows, per (head,
    position) row: max |difference| at most ``rel`` times the row's largest
    magnitude.  Deeper layers inherit the fp16 rounding of every earlier
    layer's cache (measured at most 3.5e-3 of the row maximum over the 25
    layers of the 2b shape, 2.6e-3 on the TP-8 share); a row stored at the
    wrong position or rotated by the wrong angle misses the bar by orders of
    magnitude."""
    g = k_gpu_f16.astype(np.float64)
    o = k_or.astype(np.float64)
    err = np.max(np.abs(g - o), axis=-1)
    scale = np.max(np.abs(o), axis=-1)
    bad = err > rel * scale
    assert not bad.any(), (f"{what}: {int(bad.sum())} rows off, worst relative "
                           f"{float(np.max(err / np.maximum(scale, 1e-30))):.3e}")


ROUTE_TIE = 1e-3


def compare_routing(ids_gpu: np.ndarray, ids_or: np.ndarray, router_or, top_k: int,
                    where: dict = None):
    """Routed expert ids per (position, layer), in rank order, against the oracle's.

    Where the ids differ, the GPU's choice must still be a top-k of the
    oracle's router logits r to within ``ROUTE_TIE``: its rank order is
    non-increasing in r up to the tolerance, and every chosen expert's logit
    is at least every unchosen expert's minus the tolerance (several
    routings are correct when logits are within fp32 noise of each other).
    Returns the sorted list of positions whose expert set differs (their
    outputs are not held to the bar).  Once a layer's expert set differs,
    the layers above it at that position see a different input, so they
    are not compared.  ``where`` (a dict) receives position -> that layer."""
    ids_gpu = np.asarray(ids_gpu)
    ids_or = np.asarray(ids_or)
    assert ids_gpu.shape == ids_or.shape, (ids_gpu.shape, ids_or.shape)
    tied = set()
    for i in range(ids_gpu.shape[0]):
        for l in range(ids_gpu.shape[1]):
            if i in tied:
                break
            g = ids_gpu[i, l]
            if np.array_equal(g, ids_or[i, l]):
                continue
            r = np.asarray(router_or[i][l], np.float64)
            assert len(set(g.tolist())) == top_k and np.all((g >= 0) & (g < len(r))), g
            rest = np.setdiff1d(np.arange(len(r)), g)
            order_ok = bool(np.all(r[g[:-1]] >= r[g[1:]] - ROUTE_TIE))
            set_ok = len(rest) == 0 or float(r[g].min()) >= float(r[rest].max()) - ROUTE_TIE
            assert order_ok and set_ok, (
                f"position {i} layer {l}: gpu experts {g.tolist()} != oracle "
                f"{ids_or[i, l].tolist()} (logits of gpu choice {np.round(r[g], 5).tolist()})")
            if not np.array_equal(np.sort(g), np.sort(ids_or[i, l])):
                tied.add(i)
                if where is not None:
                    where[i] = l
    return sorted(tied)


# Sampled decode.  The draw is an integer decision taken from floating point
# (keys z / T + g rounded to float32), so the kernel's token is checked
# against the oracle's sampler applied to the kernel's own logits, where the
# top-2 key margin clears the last-ulp differences of the float64 log
# (libm on the host, the device math library on the GPU); the kernel's logits
# are checked against the oracle's as for greedy decoding; and where the
# oracle's own keys have a top-2 margin wider than twice the logit tolerance
# over T, the kernel's token must also equal the oracle's own draw.
KEY_MARGIN = 1e-5


def compare_sampled_steps(z_gpu: np.ndarray, tok_gpu: np.ndarray, z_or: np.ndarray, temperature: float,
                          seed: int, pos0: int):
    from oracle.sampling import sample_keys
    n = len(tok_gpu)
    pinned = unpinned = cross = 0
    worst = 0.0
    for i in range(n):
        zo = z_or[i].astype(np.float64)
        zg = z_gpu[i].astype(np.float64)
        err = float(np.max(np.abs(zg - zo)))
        worst = max(worst, err)
        assert err <= ABS_TOL, f"step {i}: max |dz| = {err:.3e} > {ABS_TOL}"
        assert err <= REL_RANGE_TOL * float(zo.max() - zo.min()), f"step {i}: logits range"
        keys = sample_keys(z_gpu[i], temperature, seed, pos0 + i).astype(np.float64)
        order = np.argsort(-keys, kind="stable")
        top, second = keys[order[0]], keys[order[1]]
        if top - second > KEY_MARGIN * max(1.0, abs(top)):
            pinned += 1
            assert int(tok_gpu[i]) == int(order[0]), (
                f"step {i}: gpu token {int(tok_gpu[i])} != draw {int(order[0])} from the gpu logits")
        else:
            unpinned += 1
            assert int(tok_gpu[i]) in (int(order[0]), int(order[1])), f"step {i}: token not a top-2 key"
        ko = sample_keys(z_or[i], temperature, seed, pos0 + i).astype(np.float64)
        oo = np.argsort(-ko, kind="stable")
        if ko[oo[0]] - ko[oo[1]] > 2.0 * 2.0 * ABS_TOL / temperature:
            cross += 1
            assert int(tok_gpu[i]) == int(oo[0]), f"step {i}: gpu token differs from the oracle's own draw"
    return {"steps": n, "pinned": pinned, "unpinned": unpinned, "cross_checked": cross, "worst_abs": worst}


CUT_MARGIN = 1e-12     # relative float64 slack at a top-p cut (exp and rounding order)


def check_topkp_step(z_gpu: np.ndarray, tok: int, temperature: float, seed: int, pos: int, top_k: int,
                     top_p: float) -> bool:
    """The kernel's top-k / top-p draw against the oracle's, recomputed from
    the kernel's own logits.  Returns True if the step is pinned (the
    oracle's draw is unambiguous and the token equals it); otherwise the
    token must still be a draw the oracle could make within float64 slack:
    one of the two best keys over a kept set that differs from the oracle's
    by at most the candidate at the cut."""
    from oracle.sampling import MAX_TOP_K, candidate_order, kept_set, sample_keys, sample_token_topkp
    keep = kept_set(z_gpu, temperature, top_k, top_p)
    keys = sample_keys(z_gpu, temperature, seed, pos).astype(np.float64)
    kk = np.sort(keys[keep])[::-1]
    cut_close = False
    if top_p < 1.0:
        pool = candidate_order(z_gpu)[: min(top_k if top_k > 0 else MAX_TOP_K, z_gpu.shape[0])]
        z64 = np.asarray(z_gpu, np.float32).astype(np.float64)
        q = np.exp((z64[pool] - z64[pool[0]]) / float(np.float32(temperature)))
        c = np.cumsum(q)
        goal = float(np.float32(top_p)) * c[-1]
        m = len(keep)
        near = [abs(c[m - 1] - goal)] + ([abs(c[m - 2] - goal)] if m >= 2 else [])
        cut_close = min(near) <= CUT_MARGIN * goal
    key_close = len(kk) > 1 and kk[0] - kk[1] <= KEY_MARGIN * max(1.0, abs(kk[0]))
    if not cut_close and not key_close:
        assert tok == sample_token_topkp(z_gpu, temperature, seed, pos, top_k, top_p), (tok, pos)
        return True
    # the kept set may gain the candidate at the cut; the draw may be either
    # of the two best keys over it
    cand = list(kept_set(z_gpu, temperature, top_k, 1.0))[: len(keep) + 1] if cut_close else list(keep)
    order = sorted((int(i) for i in cand), key=lambda i: (-keys[i], i))
    assert tok in order[:2], (tok, pos, order[:2])
    return False
