"""Batch-1 decode benchmark on one MI355X.

A step is one decoded token: one pass of the whole hot path (embedding,
every layer's RMSNorm/QKV/RoPE+KV append/split-K attention/O/SwiGLU FFN,
final norm, lm_head, argmax and on-device feedback).  All K timed steps run
inside ONE kie_decode call, i.e. one persistent kernel launch.

Prints one JSON line: tokens/s, ms per token, the HBM roofline of the
decode kernel (algorithmic bytes per launch / launch time vs 8 TB/s), and
the CPU oracle timed on the host's cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# the files that define the decode kernel's code and parameter layout (the
# host runtime only launches it)
KERNEL_SOURCES = ("persistent_decode_monokernel_amd/csrc/kie_kernels.hip",
                  "persistent_decode_monokernel_amd/csrc/kie_params.h")
# HBM bytes of one timed decode launch, from two rocprofv3 counter passes
# (FETCH_SIZE, then WRITE_SIZE) scaled by what the same counters read for the
# streaming probe kernel of known size; the summaries with the commands are
# profiles/mono_kernel_2b_decode512.md and profiles/mono_kernel_other_workloads.md.  A figure is reported only while the
# kernel sources still hash to the digest it was measured on.
MEASURED_TRAFFIC = [
    {"sources_sha256": "43c81171fe037f4467226a6d49c0aa49b760716d55e0cf3647b0a0cfd173f0c4",
     "config": "2b", "pos0": 511, "steps": 20, "bytes": 86076204333},
    {"sources_sha256": "43c81171fe037f4467226a6d49c0aa49b760716d55e0cf3647b0a0cfd173f0c4",
     "config": "2b", "pos0": 511, "steps": 512, "bytes": 2237463797735},
    {"sources_sha256": "43c81171fe037f4467226a6d49c0aa49b760716d55e0cf3647b0a0cfd173f0c4",
     "config": "moe", "pos0": 511, "steps": 512, "bytes": 2281990157948},
    {"sources_sha256": "43c81171fe037f4467226a6d49c0aa49b760716d55e0cf3647b0a0cfd173f0c4",
     "config": "longctx", "pos0": 8191, "steps": 256, "bytes": 1099092117858},
    {"sources_sha256": "43c81171fe037f4467226a6d49c0aa49b760716d55e0cf3647b0a0cfd173f0c4",
     "config": "tp8share", "pos0": 255, "steps": 1024, "bytes": 603925445032},
]
METRIC = "batch-1 decode tokens/s + achieved HBM GB/s vs ~8 TB/s peak, ~2.2B fp16"


def source_digest() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(cfg, pos0: int, steps: int):
    digest = source_digest()
    for m in MEASURED_TRAFFIC:
        if (m["sources_sha256"], m["config"], m["pos0"], m["steps"]) == (digest, cfg.name, pos0, steps):
            return m["bytes"]
    return None


def weight_bytes_per_token(c) -> int:
    """fp16 bytes of every weight one decode step reads (active experts only)."""
    d, qd, kd = c.d_model, c.n_heads * c.head_dim, c.n_kv_heads * c.head_dim
    per_layer = (qd * d + 2 * kd * d + d * qd) + 2 * d            # attention + 2 norm gains
    if c.n_experts:
        per_layer += c.n_experts * d + (c.top_k + c.n_shared_experts) * 3 * c.expert_hidden * d
    else:
        per_layer += 3 * c.ffn_hidden * d
    total = c.n_layers * per_layer + d + c.vocab_out * d + d         # final norm, lm_head, emb row
    return 2 * total


def kv_bytes_per_position(c) -> int:
    return 2 * c.n_layers * c.n_kv_heads * c.head_dim * 2            # K and V, fp16


def decode_bytes(c, pos0: int, n: int) -> int:
    """Algorithmic HBM bytes of n decode steps starting at position pos0: all
    weights, plus at position p the p cached K/V rows read and 1 row written."""
    W = weight_bytes_per_token(c)
    kv = kv_bytes_per_position(c)
    rows = sum(p + 1 for p in range(pos0, pos0 + n))
    return n * W + kv * rows


def host_info() -> dict:
    """CPU model, usable cores and RAM of the host the CPU baseline ran on."""
    model, mem_kib = None, None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal"):
                    mem_kib = int(line.split()[1])
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)),
            "logical_cpus": os.cpu_count(),
            "ram_gib": round(mem_kib / 2**20, 1) if mem_kib else None}


def cpu_baseline(cfg, W, prompt, budget_s: float):
    """The oracle as it stands, timed on this host: decode steps after the
    workload's whole prompt (batched prefill, not timed), until about
    budget_s seconds of decode have run or the KV capacity is reached."""
    from oracle import Oracle
    from kie_synth import weights_to_numpy
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = None
    host = host_info()
    cores = host["affinity_cores"]
    Wn = weights_to_numpy(W)
    o = Oracle(cfg, Wn)
    t_pf = time.perf_counter()
    o.prefill(prompt)
    t_pf = time.perf_counter() - t_pf
    o.decode(1)                                 # widens the remaining weights once
    n = 0
    t0 = time.perf_counter()
    while True:
        o.decode(1)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or o.pos >= cfg.kv_capacity - 1:
            break
    return {"value": n / el, "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": (f"{cfg.name}: numpy fp32 oracle, {n} greedy decode steps from position "
                       f"{len(prompt) + 1} after the {len(prompt)}-token prompt's batched prefill "
                       f"({t_pf:.1f} s, not timed); {el:.1f} s of decode on {cores} usable host "
                       f"cores, BLAS threads {threads}"),
            "ms_per_token": 1e3 * el / n, "blas_threads": threads, "host": host}


def trace_summary(cfg, tr):
    """Per-stage timing of one traced decode step from the in-kernel clock
    stamps (100 MHz wall clock).  Each stage records when its inputs were
    complete ("ready"), when its main loop started ("start", after the norm
    or the RoPE and KV append) and when it finished ("end"); "wait" is ready
    minus the workgroup's previous end, "prep" start minus ready, "work" end
    minus start.  The first Q/K/V stage of a step also waits for the
    previous step's argmax barrier.  Reported per stage kind: the mean over layers of the mean
    and max over workgroups."""
    import numpy as np
    t = tr.astype(np.float64) * 10.0 / 1000.0          # ticks of 10 ns -> us
    t -= t[:, :1]
    kinds = (["qkv", "attn", "o", "router", "moe_gateup", "moe_down"] if cfg.n_experts
             else ["qkv", "attn", "o", "gateup", "down"])
    names = [k for _ in range(cfg.n_layers) for k in kinds] + ["lm_head"]
    out = {}
    prev_end = t[:, 0]
    for k, name in enumerate(names):
        if 3 + 3 * k >= t.shape[1]:
            break
        ready, start, end = t[:, 1 + 3 * k], t[:, 2 + 3 * k], t[:, 3 + 3 * k]
        parts = {"wait": ready - prev_end, "prep": start - ready, "work": end - start}
        d = out.setdefault(name, {"n": 0})
        d["n"] += 1
        for key, v in parts.items():
            d[key + "_mean_us"] = d.get(key + "_mean_us", 0.0) + float(v.mean())
            d[key + "_max_us"] = d.get(key + "_max_us", 0.0) + float(v.max())
        prev_end = end
    tot = {k: sum(d.get(k + "_mean_us", 0.0) for d in out.values()) for k in ("wait", "prep", "work")}
    for d in out.values():
        for key in list(d):
            if key != "n":
                d[key] /= d["n"]
    step = float(t[:, -1].max())
    # per step, averaged over workgroups: the time spent waiting for a
    # stage's inputs (the exchange and the step barrier) against the whole
    return {"step_us": step, "wait_us": tot["wait"], "prep_us": tot["prep"],
            "work_us": tot["work"], "idle_frac": tot["wait"] / step if step > 0 else None,
            "stages": out}


def hbm_probes(read_bytes: int = 2 << 30, copy_bytes: int = 1 << 30, reps: int = 10,
               sweep: bool = True) -> dict:
    """Achievable HBM streaming rates on this device, from the library's
    plain streaming kernel: a read-only pass over ``read_bytes`` and a copy
    of ``copy_bytes`` (reads + writes counted), in the default shape (8
    non-temporal global loads in flight per lane, four workgroups per
    compute unit); with ``sweep`` also every load kind x loads in flight x
    workgroups per compute unit, whose best read rate is the ceiling the
    decode kernel is judged against."""
    import torch
    import persistent_decode_monokernel_amd as kie
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    src = torch.empty(read_bytes // 2, dtype=torch.float16, device="cuda")
    src.fill_(1.0)
    kie.debug_stream(src, None, reps=2)
    ms_r = kie.debug_stream(src, None, reps=reps)
    out = {"read_gbs": read_bytes / (ms_r * 1e-3) / 1e9, "read_bytes": read_bytes,
           "read_ms": ms_r, "kernel": "kie::stream_kernel", "n_cu": n_cu}
    if sweep:
        pts = []
        for kind in (0, 1, 2):
            for depth in (2, 4, 8, 16):
                for per_cu in (1, 2, 4, 8):
                    kie.debug_stream(src, None, n_workgroups=per_cu * n_cu, reps=1, depth=depth,
                                     kind=kind)
                    ms = kie.debug_stream(src, None, n_workgroups=per_cu * n_cu, reps=5,
                                          depth=depth, kind=kind)
                    pts.append([kind, depth, per_cu, round(read_bytes / (ms * 1e-3) / 1e9, 1)])
        best = max(pts, key=lambda q: q[3])
        out.update({"read_best_gbs": best[3],
                    "read_best_shape": {"kind": ["global_nt", "global", "buffer_nt"][best[0]],
                                        "loads_in_flight": best[1], "wg_per_cu": best[2]},
                    "sweep_cols": ["kind(0 global nt,1 global,2 buffer nt)", "loads_in_flight",
                                   "wg_per_cu", "GB/s"],
                    "sweep": pts})
    a = src[: copy_bytes // 2]
    dst = torch.empty_like(a)
    kie.debug_stream(a, dst, reps=2)
    ms_c = kie.debug_stream(a, dst, reps=reps)
    out.update({"copy_gbs": 2 * copy_bytes / (ms_c * 1e-3) / 1e9, "copy_bytes": copy_bytes,
                "copy_ms": ms_c})
    del src, dst
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed decode steps (default: the config's)")
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--config", default="2b")
    ap.add_argument("--graph", action="store_true", help="staged per-kernel hipGraph mode")
    ap.add_argument("--reps", type=int, default=3, help="timed repetitions (median reported)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the HBM streaming probes")
    ap.add_argument("--no-trace", action="store_true",
                    help="skip the traced decode whose per-stage wait/work breakdown and idle "
                         "fraction go into detail.trace")
    ap.add_argument("--no-full", action="store_true",
                    help="skip the extra decode over the workload's whole length when --steps "
                         "is shorter")
    ap.add_argument("--no-ab", action="store_true",
                    help="skip the persistent vs staged-hipGraph comparison")
    ap.add_argument("--no-sweep", action="store_true", help="only the default streaming probe shape")
    ap.add_argument("--cooperative", action="store_true",
                    help="launch the persistent kernel as a cooperative dispatch (the default is "
                         "an ordinary dispatch, which profilers can trace; residency of every "
                         "workgroup is checked at engine creation either way)")
    ap.add_argument("--probe-only", action="store_true",
                    help="run only the HBM read/copy probes (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build measures one GPU only (batch-1 decode on a single "
              "MI355X); multi-GPU tensor parallelism is not built. Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import persistent_decode_monokernel_amd as kie
    from kie_synth import get_config, make_prompt, make_weights

    if args.probe_only:
        torch.cuda.set_device(0)
        print(json.dumps({"probe": hbm_probes(sweep=not args.no_sweep)}), flush=True)
        return 0

    cfg = get_config(args.config)
    K = args.steps if args.steps is not None else cfg.n_decode
    P = cfg.prompt_len
    max_seq = max(cfg.kv_capacity, P + max(K, args.warmup))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    W = make_weights(cfg, seed=0, device=dev)
    prompt = make_prompt(cfg, seed=0)
    stream = torch.cuda.current_stream()

    def timed(engine, n, reps):
        """Median over reps of one n-step decode call after a fresh prefill:
        (call ms from events on the engine's stream, kernel ms, prefill ms)."""
        toks = torch.empty(n, dtype=torch.int32, device=dev)
        rows = []
        for _ in range(max(1, reps)):
            engine.reset()
            engine.prefill(prompt)
            pf = engine.last_elapsed_ms()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            engine.decode_into(n, toks, None)
            e1.record(stream)
            torch.cuda.synchronize()
            rows.append((e0.elapsed_time(e1), engine.last_elapsed_ms(), pf))
        rows.sort()
        return rows[len(rows) // 2], [r[0] for r in rows]

    def make_engine(graph, trace=False):
        e = kie.Engine(cfg, W, max_seq=max_seq, graph=graph, trace=trace,
                       plain_launch=not args.cooperative)
        e.prefill(prompt)
        if args.warmup:
            e.decode(args.warmup, logits=False)
        return e

    eng = make_engine(args.graph)
    (ms, kms, pf_ms), times = timed(eng, K, args.reps)
    tok_s = K / (ms / 1e3)
    nbytes = decode_bytes(cfg, P - 1, K)
    achieved = nbytes / (kms / 1e3) / 1e9
    # the workload's whole decode length as well, when the timed K is shorter
    Kf = cfg.n_decode
    full = None
    if K != Kf and not args.no_full:
        (f_ms, f_kms, _), _ = timed(eng, Kf, args.reps)
        fb = decode_bytes(cfg, P - 1, Kf)
        full = {"steps": Kf, "ms_per_token": f_ms / Kf, "tok_s": Kf / (f_ms / 1e3),
                "kernel_ms": f_kms, "bytes": fb, "achieved_gbs": fb / (f_kms / 1e3) / 1e9,
                "frac": fb / (f_kms / 1e3) / 1e9 / HBM_PEAK_GBS,
                "traffic": measured_traffic(cfg, P - 1, Kf)}
    # the prompt through the batched (matrix-core) prefill instead: not part
    # of the decode metric, reported beside the persistent kernel's prefill
    batched_ms = None
    if not args.graph:
        eng.reset()
        eng.prefill_batched(prompt)
        eng.reset()
        eng.prefill_batched(prompt)
        batched_ms = eng.last_elapsed_ms()
    eng.close()
    # persistent kernel against the same step as one launch per stage,
    # replayed from a captured hipGraph: the cost of launching and ending a
    # kernel per stage instead of waiting on flags inside one
    ab = None
    if not args.no_ab:
        n_ab = Kf
        other = make_engine(not args.graph)
        (o_ms, o_kms, _), _ = timed(other, n_ab, args.reps)
        other.close()
        if full is not None or K == n_ab:
            mine = full["ms_per_token"] if full is not None else ms / K
        else:
            mine = None
        pers, graph = (o_ms / n_ab, mine) if args.graph else (mine, o_ms / n_ab)
        splits = max(1, max(cfg.n_kv_heads, torch.cuda.get_device_properties(0).multi_processor_count)
                     // cfg.n_kv_heads)
        per_layer = (6 if cfg.n_experts else 5) + (1 if splits > 1 else 0)
        launches = cfg.n_layers * per_layer + 2
        ab = {"steps": n_ab, "persistent_ms_per_token": pers, "graph_ms_per_token": graph,
              "graph_launches_per_token": launches,
              "extra_us_per_launch": (1e3 * (graph - pers) / launches
                                      if pers is not None and graph is not None else None)}
    trace = None
    if not args.no_trace and not args.graph:
        te = make_engine(False, trace=True)
        toks = torch.empty(8, dtype=torch.int32, device=dev)
        te.reset()
        te.prefill(prompt)
        te.decode_into(8, toks, None)
        trace = trace_summary(cfg, te.read_trace())
        trace["note"] = ("step 1 of an 8-step decode after the prompt, from the in-kernel "
                         "stamps; wait = inputs-complete minus the workgroup's previous stage "
                         "end, summed over the step's stages and averaged over workgroups")
        te.close()
    probes = None if args.no_probe else hbm_probes(sweep=not args.no_sweep)
    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": (f"{cfg.name}: {cfg.n_layers} layers, d_model {cfg.d_model}, "
                                f"{cfg.n_heads}x{cfg.head_dim} heads ({cfg.n_kv_heads} KV), "
                                + (f"MoE {cfg.n_experts}e top{cfg.top_k}+{cfg.n_shared_experts} "
                                   f"hidden {cfg.expert_hidden}" if cfg.n_experts else
                                   f"SwiGLU {cfg.ffn_hidden}")
                                + f", vocab {cfg.vocab_out}; batch 1, prompt {P}, greedy decode "
                                  f"{K}; fp16 weights N(0,0.02) seed 0, fp16 KV"),
                   "global_batch": 1, "seq_len": P + K,
                   "mode": "staged-hipgraph" if args.graph else "persistent"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(cfg, P - 1, K)},
        "detail": {"kernel": "kie::mono_kernel" if not args.graph else "kie::stage_kernel",
                   "bytes_per_launch": nbytes, "bytes_per_token": nbytes / K,
                   "kernel_ms": kms, "call_ms": ms, "reps_call_ms": times,
                   "full_decode": full, "graph_ab": ab,
                   "roofline_tok_s": HBM_PEAK_GBS * 1e9 / (nbytes / K),
                   "hbm_probe": probes,
                   "frac_of_read_probe": (achieved / probes.get("read_best_gbs", probes["read_gbs"])
                                          if probes else None),
                   "trace": trace,
                   "prefill": {"positions": P - 1,
                               "persistent_ms": pf_ms,
                               "batched_ms": batched_ms}},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, W, prompt, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
