"""bench.py's work model and driver choice (CPU only).

The byte and flop counts set every roofline fraction the bench reports, so
they are pinned here against the frame's weight shapes written out one matrix
at a time (Qwen3-TTS code predictor, rightkit-qts exporter README, "Loader
contract": per layer the fused q/k/v, output, gate, up and down projections;
fifteen lm_head matrices; the input projection W_p), not against bench.py's
own per-layer formula.
"""
import argparse
import os
import subprocess
import sys

import numpy as np

import bench
from rvq_codebook_code_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _weight_counts(g):
    """(per-step weights, layer-0 q/k/v weights, projection weights) from the
    matrix shapes [out, in]."""
    qd = g.n_q_heads * g.head_dim
    nqkv = (g.n_q_heads + 2 * g.n_kv_heads) * g.head_dim
    layer = [(nqkv, g.d_model), (g.d_model, qd), (g.d_ffn, g.d_model), (g.d_ffn, g.d_model), (g.d_model, g.d_ffn)]
    step = sum(o * i for _ in range(g.n_layers) for o, i in layer) + g.vocab * g.d_model
    return step, nqkv * g.d_model, g.d_model * g.d_talker


def test_frame_bytes_follow_the_weight_shapes():
    g = synth.WORKLOADS["b1"].geom
    step, qkv0, proj = _weight_counts(g)
    assert bench.algorithmic_bytes(g) == (15 * step + proj) * 2 == 2_426_404_864
    # with the layer-0 table: that layer's q/k/v weights at step 1 only, plus
    # one fp32 row of (nq + 2 nkv) hd values per request and step 2..15
    nqkv = (g.n_q_heads + 2 * g.n_kv_heads) * g.head_dim
    for B in (1, 2, 16):
        want = (15 * step + proj - 14 * qkv0) * 2 + 14 * B * nqkv * 4
        assert bench.algorithmic_bytes(g, B, qkv0_table=True) == want
    assert bench.algorithmic_bytes(g, 1, qkv0_table=True) == 2_309_193_728


def test_block_format_bytes():
    """Q8_0 blocks are 34 B per 32 weights, Q4_0 blocks 18 B (an f16 scale
    plus the codes)."""
    g4 = synth.WORKLOADS["q4_b1"].geom
    step, _, proj = _weight_counts(g4)
    assert bench.algorithmic_bytes(g4) == (15 * step + proj) * 18 // 32 == 682_426_368
    g8 = synth.WORKLOADS["q8ema"].geom
    step, _, proj = _weight_counts(g8)
    assert bench.algorithmic_bytes(g8) == (15 * step + proj) * 34 // 32


def test_frame_flops():
    g = synth.WORKLOADS["b128"].geom
    step, qkv0, proj = _weight_counts(g)
    assert bench.algorithmic_flops(g, 128) == 2 * 128 * (15 * step + proj)
    assert bench.algorithmic_flops(g, 128, qkv0_table=True) == 2 * 128 * (15 * step + proj - 14 * qkv0)


def test_talker_step_bytes():
    """Every Talker weight once plus the history's bf16 keys and values."""
    wl = synth.TALKER_WORKLOADS["talker_b1"]
    g = wl.geom
    qd, kd = g.n_q_heads * g.head_dim, g.n_kv_heads * g.head_dim
    mats = [(qd + 2 * kd, g.d_model), (g.d_model, qd), (g.d_ffn, g.d_model), (g.d_ffn, g.d_model),
            (g.d_model, g.d_ffn)]
    weights = (g.n_layers * sum(o * i for o, i in mats) + g.vocab * g.d_model) * 2
    kv = 1 * g.n_layers * (1024 + 1) * 2 * kd * 2
    assert bench.talker_bytes(g, 1, 1024) == weights + kv


def test_driver_choice():
    args = argparse.Namespace(sample=None, stepwise=False, generic=False)
    W = synth.WORKLOADS
    assert bench.select_driver(W["b1"].geom, 1, args) == "dataflow"
    assert bench.select_driver(W["b1"].geom, 2, args) == "dataflow"
    assert bench.select_driver(W["b16"].geom, 16, args) == "flow"
    assert bench.select_driver(W["b16"].geom, 3, args) == "flow"
    assert bench.select_driver(W["b16"].geom, 17, args) == "tiled"
    assert bench.select_driver(W["q8ema"].geom, 16, args) == "tiled"
    assert bench.select_driver(W["b128"].geom, 128, args) == "tiled"
    assert bench.select_driver(W["q4_b1"].geom, 1, args) == "dataflow"
    assert bench.select_driver(W["q8ema"].geom, 64, args) == "tiled"
    assert bench.select_driver(W["tiny_bf16"].geom, 1, args) == "tiled"
    assert bench.select_driver(W["tiny"].geom, 4, args) == "generic"
    assert bench.select_driver(W["b1"].geom, 1, argparse.Namespace(sample="0.9,50,0.95", stepwise=False,
                                                                   generic=False)) == "tiled"
    assert bench.has_qkv0_table(W["b128"].geom) and bench.has_qkv0_table(W["q4_b16"].geom)
    assert not bench.has_qkv0_table(W["tiny_bf16"].geom)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_model_flops_of_the_frame():
    """Whole-frame flops of the 1.7B geometry at B = 128: 16 positions
    through 5 layers, 15 lm_head rows, W_p once, attention over 1..16 cached
    positions (2 x 16 heads x 128 x 136 multiply-adds per layer)."""
    g = synth.WORKLOADS["b128"].geom
    per_layer = 4096 * 1024 + 1024 * 2048 + 2 * 3072 * 1024 + 1024 * 3072
    macs = 16 * 5 * per_layer + 15 * 2048 * 1024 + 1024 * 2048 + 5 * 2 * 2048 * 136
    assert macs == 1_294_630_912
    assert bench.model_flops(g, 128) == 2 * 128 * macs == 331_425_513_472


def test_timeline_analysis_on_built_stamps():
    """A hand-built frame of stamps for one layer: every phase of steps 2..15
    starts 10 us after the previous one ends, its inputs are staged 1 us (first
    workgroup) to 2 us (last) after that, and it ends 3 us (first) to 4 us
    (last) after its start; so each hand-off is 10 + 1 us, the median work 2
    us, the end spread 1 us and staged-to-last-end 3 us."""
    import numpy as np
    L = 1
    nph = 15 * (5 * L + 1)                       # phases 1..90 of steps 1..15
    T = np.zeros((4, 400, 3), dtype=np.int64)
    t = 1000.0                                   # microseconds
    for ph in range(1, nph + 1):
        s = 1 + (ph - 1) // (5 * L + 1)
        q = (ph - 1) % (5 * L + 1)
        if s >= 2 and q == 0:
            continue                             # layer 0's q/k/v: no exchange from step 2 on
        for w in range(4):
            start = t + 10.0
            T[w, ph, 0] = int(round(start * 100))
            T[w, ph, 1] = int(round((start + 1.0 + w / 3.0) * 100))
            T[w, ph, 2] = int(round((start + 3.0 + w / 3.0) * 100))
        t = t + 10.0 + 4.0
    out = bench.analyze_timeline(T, L)
    per = out["per_phase_type_us"]
    assert set(per) == {"attn", "o", "up", "down", "lm"}       # q/k/v of layer 0 never stamped after step 1
    for k, v in per.items():
        # last producer ended at prev_start + 4; first consumer staged at prev_start + 14 + 1
        assert abs(v["handoff"] - 11.0) < 1e-6, (k, v)
        assert abs(v["work_median"] - 2.0) < 1e-6
        assert abs(v["end_spread"] - 1.0) < 1e-6
        assert abs(v["ready_to_last_end"] - 3.0) < 1e-6
        assert v["phases"] == 14
    assert out["phases_with_exchange"] == nph - 14


def test_kernel_timeline_analysis_on_built_stamps():
    """The batched path's kernel timeline on hand-built stamps (100 MHz
    counter values): three launches, one stale workgroup left from before the
    frame, gaps and spans worked out by hand."""
    S = np.zeros((3, 8, 3), dtype=np.uint64)
    S[0, 0] = (1000, 0, 1500)                       # k_start: no K loop
    S[0, 1] = (1010, 0, 1520)
    S[1, 0] = (1700, 2000, 2300)                    # q/k/v product
    S[1, 1] = (1720, 2010, 2310)
    S[1, 2] = (1730, 2050, 2400)
    S[2, 0] = (500, 0, 900)                         # stale: before the frame
    S[2, 1] = (2600, 0, 3000)                       # attention
    S[2, 2] = (2650, 0, 3100)
    out = bench.analyze_kernel_timeline(S, [9, 2, 3])
    assert out["frame_span_us"] == 21.0
    assert out["kernels"] == 3
    assert out["kernel_time_us"] == 17.2
    assert out["gap_time_us"] == 3.8
    k = out["per_kernel_us"]
    assert k["start"] == {"launches": 1, "span": 5.2, "gap_before": None, "start_ramp": 0.1,
                          "workgroup_median": 5.05, "k1_median": None, "total": 5.2}
    assert k["qkv"] == {"launches": 1, "span": 7.0, "gap_before": 1.8, "start_ramp": 0.3,
                        "workgroup_median": 6.0, "k1_median": 3.0, "total": 7.0}
    assert k["attn"] == {"launches": 1, "span": 5.0, "gap_before": 2.0, "start_ramp": 0.5,
                         "workgroup_median": 4.25, "k1_median": None, "total": 5.0}


def test_free_run_agreement_counts_tokens_and_decisive_prefixes():
    """Hand-built frames: row 0 equal everywhere; row 1 differs only after its
    first non-decisive step (counts as equal up to it); row 2 differs at a
    decisive step before that."""
    t = np.arange(45, dtype=np.int64).reshape(3, 15)
    mg = np.ones((3, 15))
    mg[1, 7] = 0.01
    mg[2, 9] = 0.01
    g = t.copy()
    g[1, 10] += 1
    g[2, 3] += 1
    r = bench.free_run_agreement([g], [(t, mg, bench.DECISIVE_MARGIN)])
    assert r["frames"] == 1 and r["tokens"] == 45
    assert r["token_agreement"] == round(43 / 45, 4)
    assert r["rows_equal_to_first_non_decisive_step"] == "2/3"
    # a margin exactly at the bar is not decisive
    mg2 = np.ones((3, 15))
    mg2[2, 3] = bench.DECISIVE_MARGIN
    r2 = bench.free_run_agreement([g], [(t, mg2, bench.DECISIVE_MARGIN)])
    assert r2["rows_equal_to_first_non_decisive_step"] == "2/3"   # row 1 still differs at step 10


def test_measured_traffic_follows_the_sources(tmp_path, monkeypatch):
    """The traffic figure is read from a counter summary only while the
    sources it names hash to the recorded value."""
    import hashlib
    (tmp_path / "profiles").mkdir()
    src = tmp_path / "k.h"
    src.write_text("kernel source\n")
    h = hashlib.sha256(src.read_bytes()).hexdigest()
    (tmp_path / "profiles" / "k_tiled_b128_hbm_traffic.txt").write_text(
        "# comment: with a colon\nkernel: frame call\nsources: k.h\n"
        f"sources_sha256: {h}\ntraffic_bytes_per_launch: 12345\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("tiled", "b128") == 12345
    assert bench.measured_traffic("tiled", "b16") is None        # no summary for this workload
    assert bench.measured_traffic("generic", "b128") is None     # no summary for this driver
    src.write_text("kernel source, changed\n")
    assert bench.measured_traffic("tiled", "b128") is None
