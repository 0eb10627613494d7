"""GPU parity: the HIP decode path (through the C ABI) against the CPU oracle.

Every input is seeded and synthetic (fp16 weights ~ N(0, 0.02), uniform
prompt ids); the oracle reads host copies of the same fp16 bytes.
"""
import sys

import numpy as np
import pytest

from kie_synth import get_config, make_prompt, make_weights, weights_to_numpy
from oracle import Oracle
from tests.parity import compare_routing, compare_steps, kv_close, kv_rows_close

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


def _model(name, **kw):
    return get_config(name, **kw)


def _gpu_weights(torch, cfg, seed=0):
    return make_weights(cfg, seed=seed, device="cuda")


# ------------------------------------------------------------------- GEMV
@pytest.mark.parametrize("rows,cols", [(7680, 2560), (6912, 2560), (2560, 6912), (32768, 2560),
                                       (2560, 384), (2560, 864), (100, 72), (3, 8), (513, 1032)])
def test_gemv_stage_matches_float64(torch, kie, rows, cols):
    _say("gemv", rows, cols)
    g = torch.Generator(device="cuda")
    g.manual_seed(rows * 7 + cols)
    w = (torch.randn(rows, cols, generator=g, device="cuda") * 0.02).half()
    x = torch.randn(cols, generator=g, device="cuda")
    for n_wg in (0, 7):
        y = kie.debug_gemv(w, x, n_workgroups=n_wg).cpu().numpy().astype(np.float64)
        wn = w.cpu().numpy().astype(np.float64)
        xn = x.cpu().numpy().astype(np.float64)
        want = wn @ xn
        scale = np.abs(wn) @ np.abs(xn)
        assert np.all(np.abs(y - want) <= 1e-5 * scale + 1e-30), float(np.max(np.abs(y - want) / scale))


# ---------------------------------------------------------------- streaming probe
def test_stream_probe_copies_exactly_in_every_shape(torch, kie):
    # the probe is what the memory counters are calibrated on and what the
    # decode kernel's streaming is compared against: every load depth and
    # kind must move every byte, including a tail that is not a whole
    # grid-stride pass
    _say("stream probe shapes")
    n16 = 3 * 512 * 8 * 37 + 5
    g = torch.Generator(device="cuda").manual_seed(7)
    src = torch.randint(-2**31, 2**31 - 1, (n16 * 4,), dtype=torch.int32, device="cuda", generator=g)
    for kind in (0, 1, 2):
        for depth in (1, 2, 4, 8, 16):
            dst = torch.zeros_like(src)
            kie.debug_stream(src, dst, n_workgroups=37, reps=1, depth=depth, kind=kind)
            torch.cuda.synchronize()
            assert torch.equal(dst, src), (kind, depth)
            assert kie.debug_stream(src, None, n_workgroups=37, reps=1, depth=depth, kind=kind) > 0
    with pytest.raises(kie.KieError):
        kie.debug_stream(src, None, depth=3)
    with pytest.raises(kie.KieError):
        kie.debug_stream(src, None, kind=3)


# ---------------------------------------------------------------- barrier
def test_grid_barrier_stress(torch, kie):
    _say("barrier stress")
    viol, ms = kie.debug_barrier(0, rounds=2000)
    _say(f"barrier: {ms * 1e3:.2f} us per barrier")
    assert viol == 0


def test_grid_barrier_watchdog_forced_from_host(torch, kie):
    # a spin limit of 1 poll makes waits give up at once: the kernel must
    # report a timeout and every workgroup must leave normally
    _say("barrier watchdog")
    with pytest.raises(kie.KieError) as ei:
        kie.debug_barrier(0, rounds=50, spin_limit=1)
    assert ei.value.status == "KIE_ERR_TIMEOUT"
    viol, _ = kie.debug_barrier(0, rounds=10)      # the GPU is still fine
    assert viol == 0


# ------------------------------------------------------ end-to-end, tiny
def _run_gpu(torch, kie, cfg, W, prompt, n, **kw):
    eng = kie.Engine(cfg, W, **kw)
    eng.prefill(prompt)
    toks, logits = eng.decode(n)
    torch.cuda.synchronize()
    return eng, toks.cpu().numpy(), logits.cpu().numpy()


def _oracle_replay(cfg, Wn, prompt, toks):
    # Expert routing is an integer decision taken from floating point: for a
    # MoE model the oracle stores its KV rows in the kernel's cache precision
    # (fp16) so that both sides route from the same rounded cache.
    o = Oracle(cfg, Wn, kv_fp16=cfg.is_moe)
    o.prefill(prompt)
    _, z = o.decode(len(toks), force=toks)
    return o, z


def _check_kv(eng, o, layers, spans, exclude=()):
    """Layer 0 sees identical inputs on both sides: half an fp16 ulp.  Every
    listed layer: each row within 1e-2 of its largest magnitude.  Positions
    in ``exclude`` (an accepted MoE routing near-tie) are skipped above
    layer 0, whose rows do not depend on routing."""
    for l in layers:
        for p0, p1 in spans:
            k, v = eng.read_kv(l, p0, p1)
            if l == 0:
                # against an fp16-rounded oracle cache both sides round: 1 ulp
                u = 1.0 if o.kv_fp16 else 0.5
                kv_close(k, o.K[0][:, p0:p1], f"K layer 0 [{p0},{p1})", ulps=u)
                kv_close(v, o.V[0][:, p0:p1], f"V layer 0 [{p0},{p1})", ulps=u)
            keep = [j - p0 for j in range(p0, p1) if j not in exclude]
            kv_rows_close(k[:, keep], o.K[l][:, p0:p1][:, keep], f"K layer {l} [{p0},{p1})")
            kv_rows_close(v[:, keep], o.V[l][:, p0:p1][:, keep], f"V layer {l} [{p0},{p1})")


@pytest.mark.parametrize("mode", ["persistent", "graph", "persistent_7wg", "graph_5wg", "persistent_3wg"])
def test_tiny_decode_parity(torch, kie, mode):
    cfg = _model("tiny")
    _say("tiny parity", mode)
    W = _gpu_weights(torch, cfg)
    Wn = weights_to_numpy(W)
    prompt = make_prompt(cfg)
    kw = {"graph": mode.startswith("graph")}
    if "_" in mode:
        kw["n_workgroups"] = int(mode.split("_")[1].rstrip("wg"))
    eng, toks, z = _run_gpu(torch, kie, cfg, W, prompt, cfg.n_decode, **kw)
    assert eng.position == len(prompt) - 1 + cfg.n_decode
    o, zo = _oracle_replay(cfg, Wn, prompt, toks)
    rep = compare_steps(z, toks, zo)
    _say(mode, rep)
    assert rep["pinned"] >= cfg.n_decode // 2
    # KV cache rows (after RoPE for K) at every written position
    P = len(prompt)
    _check_kv(eng, o, range(cfg.n_layers), [(0, P - 1 + cfg.n_decode)])
    eng.close()


def test_tiny_determinism_and_composability(torch, kie):
    cfg = _model("tiny")
    _say("tiny determinism")
    W = _gpu_weights(torch, cfg)
    prompt = make_prompt(cfg)
    _, t1, z1 = _run_gpu(torch, kie, cfg, W, prompt, 40)
    _, t2, z2 = _run_gpu(torch, kie, cfg, W, prompt, 40)
    np.testing.assert_array_equal(t1, t2)
    np.testing.assert_array_equal(z1, z2)
    eng = kie.Engine(cfg, W)
    eng.prefill(prompt)
    ta, za = eng.decode(15)
    tb, zb = eng.decode(25)
    np.testing.assert_array_equal(np.concatenate([ta.cpu().numpy(), tb.cpu().numpy()]), t1)
    np.testing.assert_array_equal(np.concatenate([za.cpu().numpy(), zb.cpu().numpy()]), z1)
    # the staged (graph) mode runs the same stage code: identical bits
    _, tg, zg = _run_gpu(torch, kie, cfg, W, prompt, 40, graph=True)
    np.testing.assert_array_equal(tg, t1)
    np.testing.assert_array_equal(zg, z1)
    # reset then the same prompt again reproduces the run
    eng.reset()
    eng.prefill(prompt)
    tc, zc = eng.decode(40)
    np.testing.assert_array_equal(tc.cpu().numpy(), t1)
    eng.close()


@pytest.mark.parametrize("name", ["tiny", "moe_narrow"])
def test_trace_layout_and_results_unchanged(torch, kie, name):
    """KIE_TRACE records, for one decode step, each workgroup's clock at the
    step start and three times per stage (5 stages per dense layer, 6 per MoE
    layer, then lm_head); every workgroup's stamps are in order, and tracing
    leaves the tokens and logits bit for bit as they are."""
    cfg = _model("tiny") if name == "tiny" else _variant("moe_narrow")
    _say("trace", name)
    W = _gpu_weights(torch, cfg)
    prompt = make_prompt(cfg)
    _, t0, z0 = _run_gpu(torch, kie, cfg, W, prompt, 8)
    eng, t1, z1 = _run_gpu(torch, kie, cfg, W, prompt, 8, trace=True)
    np.testing.assert_array_equal(t1, t0)
    np.testing.assert_array_equal(z1, z0)
    tr = eng.read_trace().astype(np.int64)
    per_layer = 6 if cfg.is_moe else 5
    assert tr.shape[0] > 0 and tr.shape[1] == 1 + 3 * (cfg.n_layers * per_layer + 1), tr.shape
    assert np.all(tr[:, 0] > 0)
    assert np.all(np.diff(tr, axis=1) >= 0)
    eng.close()


def test_tiny_edge_cases(torch, kie):
    cfg = _model("tiny")
    _say("tiny edges")
    W = _gpu_weights(torch, cfg)
    Wn = weights_to_numpy(W)
    # a one-token prompt (nothing to prefill) and the last position of the cache
    prompt = make_prompt(cfg, length=1)
    eng, toks, z = _run_gpu(torch, kie, cfg, W, prompt, 5, max_seq=5)
    o, zo = _oracle_replay(cfg.with_(max_seq=5), Wn, prompt, toks)
    compare_steps(z, toks, zo)
    with pytest.raises(kie.KieError) as ei:
        eng.decode(1)
    assert ei.value.status == "KIE_ERR_CONTEXT_OVERFLOW"
    with pytest.raises(kie.KieError) as ei:
        eng.prefill(prompt)
    assert ei.value.status == "KIE_ERR_BAD_STATE"
    eng.reset()
    with pytest.raises(kie.KieError) as ei:
        eng.prefill([cfg.vocab_in])
    assert ei.value.status == "KIE_ERR_TOKEN_RANGE"
    with pytest.raises(kie.KieError) as ei:
        eng.decode(1)
    assert ei.value.status == "KIE_ERR_BAD_STATE"
    toks0, _ = eng.decode(0)                  # no-op
    assert toks0.numel() == 0
    # a host pointer is refused before any launch
    import torch as t
    with pytest.raises(kie.KieError) as ei:
        eng.prefill(prompt)
        eng.decode_into(1, t.empty(1, dtype=t.int32))
    assert ei.value.status == "KIE_ERR_INVALID_ARG"
    eng.close()


def test_tiny_weights_too_small_rejected(torch, kie):
    cfg = _model("tiny")
    W = _gpu_weights(torch, cfg)
    W["lm_head"] = W["lm_head"][: cfg.vocab_out // 2].clone()
    with pytest.raises(kie.KieError) as ei:
        kie.Engine(cfg, W)
    assert ei.value.status == "KIE_ERR_INVALID_ARG"


# ------------------------------------------------------ end-to-end, 2.2B
@pytest.mark.timeout(900)
def test_2b_full_replay(torch, kie):
    """The ~2.2B model at full size in the launch the benchmark times:
    prompt 512, then 512 greedy decode steps in ONE kie_decode call (positions
    511..1022, where the context-sized split count grows from 4 to 8 per KV
    head).  The oracle replays every step teacher-forced on the kernel's
    tokens; every step is held to the logit and token bar, and K/V rows of
    three layers are checked at positions across the prompt and the decode."""
    cfg = _model("2b")
    _say("2b full replay: weights")
    W = _gpu_weights(torch, cfg)
    prompt = make_prompt(cfg)
    n = cfg.n_decode
    _say("2b full replay: gpu run")
    eng, toks, z = _run_gpu(torch, kie, cfg, W, prompt, n)
    assert eng.position == len(prompt) - 1 + n
    _say("2b full replay: oracle replay of", n, "steps")
    Wn = weights_to_numpy(W)
    o, zo = _oracle_replay(cfg, Wn, prompt, toks)
    rep = compare_steps(z, toks, zo)
    _say("2b full replay", rep)
    assert rep["pinned"] >= n // 2
    P = len(prompt)
    _check_kv(eng, o, (0, 12, 24),
              [(0, 1), (255, 256), (P - 2, P - 1), (600, 601), (800, 801), (P - 1 + n - 2, P - 1 + n)])
    eng.close()


def test_occupancy_is_checked_at_create(torch, kie):
    """A grid that cannot be co-resident is refused by kie_create, before
    any launch: the decode kernel fits one workgroup per compute unit, so 32
    more workgroups than compute units must fail with KIE_ERR_OCCUPANCY
    (a far larger grid fails earlier, on the LDS its attention splits
    need)."""
    cfg = _model("tiny")
    W = _gpu_weights(torch, cfg)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    with pytest.raises(kie.KieError) as ei:
        kie.Engine(cfg, W, n_workgroups=n_cu + 32)
    assert ei.value.status == "KIE_ERR_OCCUPANCY"


def test_argmax_exact_ties_pick_the_lowest_index(torch, kie):
    """Rows of lm_head that are bit-identical give bit-identical logits, so
    the greedy token faces exact ties.  Rows 7 and 3001 hold +8 r and rows 9
    and 2000 hold -8 r for a random row r, every other row is zero: each step
    the maximum is shared by two rows (7 and 3001 when r.h > 0, else 9 and
    2000) and the token must be the lower of the two.  Then every lm_head row
    equal: all logits tie and the token must be 0 at every step."""
    cfg = _model("tiny")
    _say("argmax ties")
    W = _gpu_weights(torch, cfg)
    prompt = make_prompt(cfg)
    r = W["lm_head"][5].float()
    lm = torch.zeros_like(W["lm_head"])
    lm[7] = lm[3001] = (8.0 * r).half()
    lm[9] = lm[2000] = (-8.0 * r).half()
    W2 = dict(W)
    W2["lm_head"] = lm.contiguous()
    n = 16
    eng, toks, z = _run_gpu(torch, kie, cfg, W2, prompt, n)
    for i in range(n):
        assert z[i][7] == z[i][3001] and z[i][9] == z[i][2000], i
        want = 7 if z[i][7] > 0 else 9
        assert z[i][want] == z[i].max()
        assert toks[i] == want, (i, toks[i], want)
    # the logits themselves against the oracle (tied steps are unpinned)
    o, zo = _oracle_replay(cfg, weights_to_numpy(W2), prompt, toks)
    compare_steps(z, toks, zo)
    eng.close()
    W3 = dict(W)
    W3["lm_head"] = W["lm_head"][11:12].expand_as(W["lm_head"]).contiguous()
    eng, toks, z = _run_gpu(torch, kie, cfg, W3, prompt, n)
    assert np.all(z == z[:, :1]), "identical rows must give identical logits"
    np.testing.assert_array_equal(toks, np.zeros(n, np.int32))
    eng.close()


# ------------------------------------------- the other workload shapes
# Reduced depth keeps the oracle's replay to seconds; widths, head layout,
# vocabulary split and expert counts are those of the full workloads.
VARIANTS = {
    # one tensor-parallel-8 share run standalone: 3 heads x 128, FFN 864,
    # 32768-row embedding but a 4096-row lm_head
    "tp8share_3l": dict(name="tp8share", n_layers=3, prompt_len=96, n_decode=32),
    # grouped-query attention, 32 query heads x 80 over 8 KV heads, a
    # prompt long enough that every attention split holds many positions
    "longctx_2l": dict(name="longctx", n_layers=2, prompt_len=1200, n_decode=16),
    # 64 routed experts (top 6, softmax weights) + 2 shared, hidden 1408
    "moe_2l": dict(name="moe", n_layers=2, prompt_len=48, n_decode=24),
    # a narrow MoE with few experts: many routing decisions per second of oracle
    "moe_narrow": dict(name="moe", n_layers=2, d_model=256, n_heads=4, n_kv_heads=4,
                       head_dim=64, vocab_in=4096, vocab_out=4096, n_experts=8, top_k=2,
                       n_shared_experts=1, expert_hidden=128, prompt_len=64, n_decode=48),
    # the same narrow MoE with the selected experts' weights rescaled to sum to 1
    "moe_narrow_renorm": dict(name="moe", n_layers=2, d_model=256, n_heads=4, n_kv_heads=4,
                              head_dim=64, vocab_in=4096, vocab_out=4096, n_experts=8, top_k=2,
                              n_shared_experts=1, expert_hidden=128, prompt_len=64, n_decode=48,
                              moe_renorm=True),
    # GQA with two query heads per KV head and a head size of 64
    "gqa2_narrow": dict(name="tiny", n_heads=8, n_kv_heads=4, head_dim=32, prompt_len=80,
                        n_decode=40),
    # the MoE build with grouped query heads: 2 and 4 query heads per KV head
    # (the matrix-core attention), head size 32
    "moe_gqa2_narrow": dict(name="moe", n_layers=2, d_model=256, n_heads=8, n_kv_heads=4,
                            head_dim=32, vocab_in=4096, vocab_out=4096, n_experts=8, top_k=2,
                            n_shared_experts=1, expert_hidden=128, prompt_len=64, n_decode=32),
    "moe_gqa4_narrow": dict(name="moe", n_layers=2, d_model=256, n_heads=8, n_kv_heads=2,
                            head_dim=32, vocab_in=4096, vocab_out=4096, n_experts=8, top_k=2,
                            n_shared_experts=1, expert_hidden=128, prompt_len=64, n_decode=32),
}


def _variant(key):
    kw = dict(VARIANTS[key])
    return _model(kw.pop("name"), **kw)


def _moe_check(eng, o, cfg, positions):
    """Routing at every listed position (prefill and decode) against the
    oracle; returns the positions with an accepted near-tie difference."""
    positions = list(positions)
    ids = np.concatenate([eng.expert_ids(p, p + 1) for p in positions])
    ids_or = np.stack([o.route[p][0] for p in positions])
    r_or = [o.route[p][1] for p in positions]
    where = {}
    tied = [positions[i] for i in compare_routing(ids, ids_or, r_or, cfg.top_k, where)]
    _say("routing near-ties (position: layer)", {positions[i]: l for i, l in where.items()})
    return tied


@pytest.mark.parametrize("key", sorted(VARIANTS))
def test_variant_decode_parity(torch, kie, key):
    cfg = _variant(key)
    _say("variant parity", key)
    W = _gpu_weights(torch, cfg)
    Wn = weights_to_numpy(W)
    prompt = make_prompt(cfg)
    n = cfg.n_decode
    eng, toks, z = _run_gpu(torch, kie, cfg, W, prompt, n)
    assert eng.position == len(prompt) - 1 + n
    assert np.all((toks >= 0) & (toks < cfg.vocab_out))
    o, zo = _oracle_replay(cfg, Wn, prompt, toks)
    P = len(prompt)
    tied = _moe_check(eng, o, cfg, range(P - 1 + n)) if cfg.is_moe else []
    rep = compare_steps(z, toks, zo, skip=[q - (P - 1) for q in tied if q >= P - 1])
    _say(key, rep, "routing near-ties at positions", tied)
    # not vacuous: enough steps clear the top-2 margin for the token check
    assert rep["pinned"] >= max(4, n // 4)
    _check_kv(eng, o, range(cfg.n_layers), [(0, P - 1 + n)], exclude=tied)
    eng.close()


# Grouped-query attention shapes: the matrix-core form (head size a multiple
# of 16 up to 80) at several head sizes and group sizes, a small grid (so a
# split holds several 32-position tiles per wave, or a workgroup runs several
# units), and the vector form that a wider head keeps.
GQA_SHAPES = {
    "g2_hd16": dict(n_heads=8, n_kv_heads=4, head_dim=16, n_workgroups=0, prompt_len=90),
    "g4_hd48": dict(n_heads=8, n_kv_heads=2, head_dim=48, n_workgroups=0, prompt_len=90),
    "g2_hd64_tiles": dict(n_heads=4, n_kv_heads=2, head_dim=64, n_workgroups=4, prompt_len=700),
    "g4_hd80_units": dict(n_heads=16, n_kv_heads=4, head_dim=80, n_workgroups=3, prompt_len=150),
    "g2_hd128_vector": dict(n_heads=4, n_kv_heads=2, head_dim=128, n_workgroups=64, prompt_len=90),
}


@pytest.mark.parametrize("key", sorted(GQA_SHAPES))
def test_grouped_attention_shapes(torch, kie, key):
    kw = dict(GQA_SHAPES[key])
    nwg = kw.pop("n_workgroups")
    cfg = _model("tiny", n_layers=2, n_decode=24, **kw)
    _say("grouped attention", key)
    W = _gpu_weights(torch, cfg)
    prompt = make_prompt(cfg)
    n = cfg.n_decode
    extra = {"n_workgroups": nwg} if nwg else {}
    eng, toks, z = _run_gpu(torch, kie, cfg, W, prompt, n, **extra)
    o, zo = _oracle_replay(cfg, weights_to_numpy(W), prompt, toks)
    rep = compare_steps(z, toks, zo)
    _say(key, rep)
    assert rep["pinned"] >= n // 4
    P = len(prompt)
    _check_kv(eng, o, (0, 1), [(0, 8), (P - 40, P - 1 + n)])
    eng.close()
    # the staged mode runs the same units one stage per kernel: same bits
    eg, tg, zg = _run_gpu(torch, kie, cfg, W, prompt, n, graph=True, **extra)
    np.testing.assert_array_equal(tg, toks)
    np.testing.assert_array_equal(zg, z)
    eg.close()


def test_gqa_merge_with_fewer_splits_than_heads(torch, kie):
    """Grouped-query attention (4 query heads per KV head) at positions
    199..298, where the context-sized split count is 2, then 3: fewer splits
    than query heads, so one merging workgroup merges several heads (split s
    takes heads s, s + S, ...).  The staged mode, whose merge kernel gives
    every query head its own workgroup, must give the same bits."""
    cfg = _model("longctx", n_layers=2, prompt_len=200, n_decode=100)
    _say("gqa fewer splits than heads")
    W = _gpu_weights(torch, cfg)
    prompt = make_prompt(cfg)
    n = cfg.n_decode
    eng, toks, z = _run_gpu(torch, kie, cfg, W, prompt, n)
    o, zo = _oracle_replay(cfg, weights_to_numpy(W), prompt, toks)
    rep = compare_steps(z, toks, zo)
    _say("gqa fewer splits", rep)
    assert rep["pinned"] >= n // 2
    P = len(prompt)
    _check_kv(eng, o, (0, 1), [(0, 8), (P - 2, P - 1 + n)])
    eng.close()
    eg, tg, zg = _run_gpu(torch, kie, cfg, W, prompt, n, graph=True)
    np.testing.assert_array_equal(tg, toks)
    np.testing.assert_array_equal(zg, z)
    eg.close()


def test_longctx_8192_prompt_attention(torch, kie):
    """The long-context head layout (GQA 32 x 80 over 8 KV heads) with the
    full 8192-token prompt and the full cache capacity, so the split-K
    attention runs over its real span; two layers keep the oracle's batched
    prefill to seconds."""
    cfg = _model("longctx", n_layers=2, n_decode=8)
    _say("longctx 8192: weights")
    W = _gpu_weights(torch, cfg)
    prompt = make_prompt(cfg)
    n = cfg.n_decode
    _say("longctx 8192: gpu run")
    eng, toks, z = _run_gpu(torch, kie, cfg, W, prompt, n, max_seq=8192 + 256)
    _say("longctx 8192: oracle replay")
    o, zo = _oracle_replay(cfg.with_(max_seq=8192 + 256), weights_to_numpy(W), prompt, toks)
    rep = compare_steps(z, toks, zo)
    _say("longctx 8192", rep)
    P = len(prompt)
    _check_kv(eng, o, (0, 1), [(0, 64), (4000, 4100), (P - 80, P - 1 + n)])
    eng.close()


@pytest.mark.parametrize("name,prompt_len,n,layers", [
    ("tp8share", 256, 8, (0, 12, 24)),
    ("longctx", 256, 6, (0, 12, 24)),
    # all 25 layers over a 2048-token prompt: splits of ~120 positions, several
    # 32-position tiles of the matrix-core attention per split
    ("longctx", 2048, 6, (0, 12, 24)),
    ("moe", 8, 4, (0, 11, 23)),
])
def test_full_size_variant_parity_sampled(torch, kie, name, prompt_len, n, layers):
    """Each other workload at full depth and width, with the cache capacity
    of its full run (so the attention split layout is the real one), on a
    prompt short enough for the oracle to replay every step."""
    full = _model(name)
    cfg = full.with_(prompt_len=prompt_len, n_decode=n)
    cap = full.prompt_len + full.n_decode
    _say(f"{name} full size: weights")
    W = _gpu_weights(torch, cfg)
    prompt = make_prompt(cfg)
    _say(f"{name} full size: gpu run")
    eng, toks, z = _run_gpu(torch, kie, cfg, W, prompt, n, max_seq=cap)
    _say(f"{name} full size: oracle replay")
    o = Oracle(cfg.with_(max_seq=cap), weights_to_numpy(W), cache_bytes=24 << 30,
               kv_fp16=cfg.is_moe)
    o.prefill(prompt)
    _, zo = o.decode(n, force=toks)
    P = len(prompt)
    tied = _moe_check(eng, o, cfg, range(P - 1 + n)) if cfg.is_moe else []
    rep = compare_steps(z, toks, zo, skip=[q - (P - 1) for q in tied if q >= P - 1])
    _say(name, rep, "routing near-ties at positions", tied)
    _check_kv(eng, o, layers, [(0, 1), (P // 2, P // 2 + 1), (P - 1, P - 1 + n)], exclude=tied)
    eng.close()


@pytest.mark.timeout(900)
def test_moe_full_depth_prompt_512(torch, kie):
    """The MoE workload at full depth and width with its real prompt of 512
    tokens, then 128 decode steps; the oracle replays all of them (the first
    128 decode steps of the 512-step run).  Routing is compared at every
    prompt and decode position."""
    cfg = _model("moe")
    n = 128
    cap = cfg.prompt_len + cfg.n_decode
    _say("moe full depth 512: weights")
    W = _gpu_weights(torch, cfg)
    prompt = make_prompt(cfg)
    _say("moe full depth 512: gpu run")
    eng, toks, z = _run_gpu(torch, kie, cfg, W, prompt, n, max_seq=cap)
    _say("moe full depth 512: oracle replay")
    o = Oracle(cfg.with_(max_seq=cap), weights_to_numpy(W), cache_bytes=96 << 30, kv_fp16=True)
    o.prefill(prompt)
    _, zo = o.decode(n, force=toks)
    P = len(prompt)
    tied = _moe_check(eng, o, cfg, range(P - 1 + n))
    rep = compare_steps(z, toks, zo, skip=[q - (P - 1) for q in tied if q >= P - 1])
    _say("moe full depth 512", rep, "routing near-ties at positions", tied)
    assert rep["pinned"] >= n // 2
    _check_kv(eng, o, (0, 11, 23), [(0, 1), (P // 2, P // 2 + 1), (P - 1, P - 1 + n)], exclude=tied)
    eng.close()
