"""Host-side logic of bench.py (no GPU): the algorithmic byte count behind
the roofline, the per-stage trace breakdown and idle fraction, the guard on
counter-measured traffic, and the refusal of a multi-GPU run."""
import numpy as np

import bench
from kie_synth import get_config


def test_decode_bytes_is_weights_plus_cache_rows():
    c = get_config("tiny")
    d, qd, kd, F = c.d_model, c.n_heads * c.head_dim, c.n_kv_heads * c.head_dim, c.ffn_hidden
    per_layer = qd * d + 2 * kd * d + d * qd + 2 * d + 3 * F * d
    weights = 2 * (c.n_layers * per_layer + d + c.vocab_out * d + d)
    assert bench.weight_bytes_per_token(c) == weights
    row = 2 * c.n_layers * c.n_kv_heads * c.head_dim * 2          # K and V, fp16, every layer
    # three steps from position 10: positions 10, 11, 12 read 11, 12, 13 rows (with their own)
    assert bench.decode_bytes(c, 10, 3) == 3 * weights + row * (11 + 12 + 13)


def test_moe_bytes_count_only_active_experts():
    c = get_config("moe")
    dense_part = c.n_heads * c.head_dim * c.d_model * 2 + 2 * c.n_kv_heads * c.head_dim * c.d_model
    expert = 3 * c.expert_hidden * c.d_model
    per_layer = dense_part + 2 * c.d_model + c.n_experts * c.d_model + \
        (c.top_k + c.n_shared_experts) * expert
    want = 2 * (c.n_layers * per_layer + 2 * c.d_model + c.vocab_out * c.d_model)
    assert bench.weight_bytes_per_token(c) == want


def test_trace_summary_splits_wait_prep_work():
    c = get_config("tiny", n_layers=1)
    # two workgroups, one layer (5 stages) + lm_head: 1 + 3 * 6 stamps of 10 ns ticks
    n_ev = 1 + 3 * 6
    tr = np.zeros((2, n_ev), dtype=np.uint64)
    for w in range(2):
        t = 1000 + 7 * w                    # the step start differs per workgroup
        tr[w, 0] = t
        for k in range(6):
            wait, prep, work = 100 * (k + 1), 10 + w, 50
            t += wait
            tr[w, 1 + 3 * k] = t
            t += prep
            tr[w, 2 + 3 * k] = t
            t += work
            tr[w, 3 + 3 * k] = t
    s = bench.trace_summary(c, tr)
    # 10 ns ticks -> us: wait of stage k is (k + 1) us, prep 0.10 / 0.11 us, work 0.5 us
    assert abs(s["stages"]["qkv"]["wait_mean_us"] - 1.0) < 1e-9
    assert abs(s["stages"]["lm_head"]["wait_mean_us"] - 6.0) < 1e-9
    assert abs(s["stages"]["attn"]["prep_mean_us"] - 0.105) < 1e-9
    assert abs(s["stages"]["attn"]["prep_max_us"] - 0.11) < 1e-9
    assert abs(s["wait_us"] - 21.0) < 1e-9
    assert abs(s["work_us"] - 3.0) < 1e-9
    step = 21.0 + 6 * 0.11 + 3.0                                   # the slower workgroup
    assert abs(s["step_us"] - step) < 1e-9
    assert abs(s["idle_frac"] - 21.0 / step) < 1e-12


def test_measured_traffic_needs_the_same_sources_and_launch():
    c = get_config("2b")
    digest = bench.source_digest()
    saved = list(bench.MEASURED_TRAFFIC)
    try:
        bench.MEASURED_TRAFFIC[:] = [{"sources_sha256": digest, "config": "2b", "pos0": 511,
                                      "steps": 20, "bytes": 123},
                                     {"sources_sha256": "0" * 64, "config": "2b", "pos0": 511,
                                      "steps": 512, "bytes": 456}]
        assert bench.measured_traffic(c, 511, 20) == 123
        assert bench.measured_traffic(c, 511, 512) is None      # measured on other sources
        assert bench.measured_traffic(c, 510, 20) is None       # another launch
    finally:
        bench.MEASURED_TRAFFIC[:] = saved


def test_host_info_reports_the_usable_cores():
    import os
    h = bench.host_info()
    assert h["affinity_cores"] == len(os.sched_getaffinity(0))
    assert h["ram_gib"] is None or h["ram_gib"] > 0


def test_multi_gpu_run_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
