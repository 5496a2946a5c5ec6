"""Benchmark of the code-predictor loop on one MI355X.

One step = one frame of the whole hot path (projection, 15 greedy steps of
the 5-layer predictor with lm_head argmax and embedding accumulation) for all
B requests of the workload, i.e. one qp_run_frames call.  Inputs are seeded
synthetic tensors already resident in HBM; weights are seeded synthetic draws
with the 1.7B predictor's shapes.

Prints one JSON line: frames/s (whole job), the roofline of the frame kernel
(algorithmic weight bytes per frame-batch over the measured time per launch,
against 8 TB/s HBM; at B = 128 flops against the bf16 matrix-core peak) and
the CPU oracle's own rate on a bounded sample.  The metric is quoted at B = 1,
16 and 128: the default run's line is the B = 1 workload, and it carries the
B = 16 and B = 128 workloads, timed in the same run, under "workloads".

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload b1] [--only]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from rvq_codebook_code_amd import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "code-predictor frames/sec (15 tokens each) at B=1/16/128; % HBM/MFMA roofline"


def bytes_per_weight(dtype: str) -> float:
    return {"f32": 4.0, "bf16": 2.0, "q8_0": 34.0 / 32.0, "q4_0": 18.0 / 32.0}[dtype]


def algorithmic_bytes(g: synth.Geometry, B: int = 1, qkv0_table: bool = False) -> int:
    """Weights the method must stream per frame-batch: every layer matrix and
    one lm_head per step (15 steps), plus the projection once per frame.  The
    gathered embedding rows (B*16 rows) are left out: a lower bound.

    qkv0_table: the driver reads layer 0's q/k/v rows of steps 2..15 from the
    create-time table (B fp32 rows per step) instead of streaming layer 0's
    q/k/v weights, so those weights count once, not 15 times."""
    qd = g.n_q_heads * g.head_dim
    nqkv = (g.n_q_heads + 2 * g.n_kv_heads) * g.head_dim
    per_layer = nqkv * g.d_model + g.d_model * qd + 2 * g.d_ffn * g.d_model + g.d_model * g.d_ffn
    per_step = g.n_layers * per_layer + g.vocab * g.d_model
    bpw = bytes_per_weight(g.weight_dtype)
    total = 15 * per_step * bpw + g.d_model * g.d_talker * bpw
    if qkv0_table:
        total += 14 * (B * nqkv * 4 - nqkv * g.d_model * bpw)
    return int(round(total))


def algorithmic_flops(g: synth.Geometry, B: int, qkv0_table: bool = False) -> int:
    """2 flops per weight per request row (15 steps; the prefill's extra row
    and attention are left out).  qkv0_table: layer 0's q/k/v product runs at
    step 1 only (see algorithmic_bytes)."""
    qd = g.n_q_heads * g.head_dim
    nqkv = (g.n_q_heads + 2 * g.n_kv_heads) * g.head_dim
    per_layer = nqkv * g.d_model + g.d_model * qd + 2 * g.d_ffn * g.d_model + g.d_model * g.d_ffn
    per_step = g.n_layers * per_layer + g.vocab * g.d_model
    total = 15 * per_step + g.d_model * g.d_talker
    if qkv0_table:
        total -= 14 * nqkv * g.d_model
    return 2 * B * total


def model_flops(g: synth.Geometry, B: int) -> int:
    """The frame's whole arithmetic, independent of how a driver reduces it:
    all 16 positions (the prefill's two and one per later step) through the
    layers, 15 lm_head rows, the projection of H, and attention's scores and
    weighted values over the cached positions (2 flops per multiply-add)."""
    qd = g.n_q_heads * g.head_dim
    nqkv = (g.n_q_heads + 2 * g.n_kv_heads) * g.head_dim
    per_layer = nqkv * g.d_model + g.d_model * qd + 2 * g.d_ffn * g.d_model + g.d_model * g.d_ffn
    attn = g.n_layers * 2 * qd * sum(p + 1 for p in range(16))
    macs = 16 * g.n_layers * per_layer + 15 * g.vocab * g.d_model + g.d_model * g.d_talker + attn
    return 2 * B * macs


def has_qkv0_table(g: synth.Geometry) -> bool:
    """The library builds the layer-0 q/k/v table for the 1.7B geometry with
    bf16, Q8_0 or Q4_0 weights (the handles the dataflow driver can run)."""
    return (g.weight_dtype in ("bf16", "q8_0", "q4_0") and 1 <= g.n_layers <= 5 and
            all(getattr(g, k) == v for k, v in _DATAFLOW_GEOMETRY.items()))


TALKER_METRIC = "Talker decode steps/sec (H and q0 per request) at a 1024-position history; % HBM roofline"


def talker_bytes(g, B: int, ctx: int) -> int:
    """Bytes one Talker step must move: every weight once (the codec head
    included) plus each request's cached keys and values (bf16) of the ctx
    positions it attends over, and the new position's key and value."""
    qd, kd = g.n_q_heads * g.head_dim, g.n_kv_heads * g.head_dim
    per_layer = g.d_model * (qd + 2 * kd) + qd * g.d_model + 3 * g.d_model * g.d_ffn
    weights = int((g.n_layers * per_layer + g.vocab * g.d_model) * bytes_per_weight(g.weight_dtype))
    kv = B * g.n_layers * (ctx + 1) * 2 * kd * 2
    return weights + kv


def run_talker(args, torch, dev):
    from oracle import talker as TK
    from rvq_codebook_code_amd import binding as bd
    wl = synth.TALKER_WORKLOADS[args.workload]
    g, B, ctx = wl.geom, wl.batch, wl.context
    W = synth.make_talker_weights(g, wl.weight_seed)
    steps = args.steps + args.warmup
    tk = bd.Talker(W, g, max_batch=B, n_slots=B, max_ctx=ctx + steps + 1)
    K, V = synth.make_talker_history(g, ctx, wl.input_seed + 1)
    Kd = torch.from_numpy(K.view(np.int16)).to(dev)
    Vd = torch.from_numpy(V.view(np.int16)).to(dev)
    for b in range(B):
        tk.load_history(b, Kd, Vd)
    del Kd, Vd
    X = torch.from_numpy(synth.make_talker_inputs(g, B, 16, wl.input_seed)).to(dev)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    H = torch.zeros((B, g.d_model), device=dev)
    q0 = torch.zeros((B,), dtype=torch.int32, device=dev)
    posd = [torch.full((B,), ctx + i, dtype=torch.int32, device=dev) for i in range(steps)]
    for i in range(args.warmup):
        tk.step(X[i % 16], slots, posd[i], ctx + i + 1, H, q0)
    torch.cuda.synchronize()
    if tk.get_error():
        raise RuntimeError("device flag raised during warm-up")
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.warmup, steps):
        tk.step(X[i % 16], slots, posd[i], ctx + i + 1, H, q0)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    if tk.get_error():
        raise RuntimeError("device flag raised during the timed steps")
    ms_per_step = ms / args.steps
    mid = ctx + args.warmup + args.steps // 2          # mean history over the timed steps
    nbytes = talker_bytes(g, B, mid)
    achieved = nbytes / (ms_per_step / 1e3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        threads, host = host_cores()
        model = TK.TalkerOracle(W, g, keep=True)
        Kf = (K.astype(np.uint32) << 16).view(np.float32).astype(np.float64)[:, :ctx]
        Vf = (V.astype(np.uint32) << 16).view(np.float32).astype(np.float64)[:, :ctx]
        Xh = X.cpu().numpy()
        t0 = time.perf_counter()
        n = 0
        while True:
            TK.decode_step(model, Xh[n % 16, 0], ctx, Kf, Vf)
            n += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_budget or n >= 64:
                break
        cpu = {"value": round(n / el, 4), "unit": "steps/s", "cores": int(threads), "kind": "oracle", "host": host,
               "sample": f"{n} decode step(s) of 1 request at a {ctx}-position history, fp64 NumPy, "
                         f"{el:.1f} s (after materialising the weights)"}
    line = {
        "metric": TALKER_METRIC,
        "value": round(B * args.steps / (ms / 1e3), 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "history": ctx,
                   "talker": f"d={g.d_model} L={g.n_layers} heads={g.n_q_heads}/{g.n_kv_heads}x{g.head_dim} "
                             f"F={g.d_ffn} V={g.vocab}",
                   "weights": g.weight_dtype, "algorithmic_bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    tk.close()


def host_cores():
    """BLAS threads the oracle's products use, the host's CPU count and the
    CPUs this process may run on."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    try:
        nproc = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        nproc = os.cpu_count()
    return int(threads), {"blas_threads": int(threads), "os_cpu_count": os.cpu_count(), "nproc": nproc}


def cpu_baseline(wl, W, H, q0, budget_s: float, sampling=None, U=None):
    """The oracle as it stands, on the host, for about ``budget_s`` seconds of
    frames of the same workload (sampled frames when ``sampling`` is given)."""
    from oracle import predictor as O
    threads, host = host_cores()
    model = O.OracleModel(W, wl.geom)
    B = H.shape[1]
    n = 0
    outs = []
    t0 = time.perf_counter()
    while True:
        if sampling is None:
            r = O.run_frames(model, H[n % H.shape[0]], q0[n % H.shape[0]])
        else:
            r = O.run_frames(model, H[n % H.shape[0]], q0[n % H.shape[0]], sampling=sampling, uniforms=U[n % H.shape[0]])
        # sampled frames: a draw is decisive when its uniform is not within
        # 1e-5 (relative) of a boundary of the cumulative distribution
        outs.append((r["tokens"], r["margin"], DECISIVE_MARGIN) if sampling is None
                    else (r["tokens"], r["sample_margin"], SAMPLE_DECISIVE_MARGIN))
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= H.shape[0]:
            break
    return {"value": round(n * B / el, 3), "unit": "frames/s", "cores": int(threads),
            "kind": "oracle", "host": host,
            "sample": f"{n} frame(s) of {B} request(s) of the {wl.name} workload"
                      f"{' (sampled)' if sampling else ''}, fp64 NumPy, {el:.1f} s"}, outs


# a step is decisive when the oracle's top-2 logit margin exceeds this (the
# bar under which greedy tokens must match bit for bit); for a sampled draw,
# when its relative margin to the nearest boundary exceeds the second
DECISIVE_MARGIN = 0.05
SAMPLE_DECISIVE_MARGIN = 1e-5


def free_run_agreement(gpu_tokens, oracle_outs):
    """Token agreement of free-running GPU frames with the oracle's free run
    of the same frames: over all tokens, and per row up to its first step
    that is not decisive (where the two must agree)."""
    import numpy as np
    tot = same = rows = rows_ok = 0
    for g, (t, mg, thr) in zip(gpu_tokens, oracle_outs):
        g = np.asarray(g, dtype=np.int64)
        tot += g.size
        same += int((g == t).sum())
        for b in range(g.shape[0]):
            nd = np.nonzero(mg[b] <= thr)[0]
            k = int(nd[0]) if nd.size else g.shape[1]
            rows += 1
            rows_ok += int(np.array_equal(g[b, :k], t[b, :k]))
    return {"frames": len(oracle_outs), "tokens": tot, "token_agreement": round(same / max(tot, 1), 4),
            "rows_equal_to_first_non_decisive_step": f"{rows_ok}/{rows}"}


COPY_BYTES = 1 << 30

_DATAFLOW_GEOMETRY = dict(d_talker=2048, d_model=1024, n_q_heads=16, n_kv_heads=8, head_dim=128,
                          d_ffn=3072, vocab=2048)


def select_driver(g, B: int, args) -> str:
    """The driver the library picks for this call (same rule as the C side)."""
    if getattr(args, "sample", None):
        return "tiled"
    if args.stepwise:
        return "stepwise"
    if args.generic:
        return "generic"
    if getattr(args, "flow", False):
        return "flow"
    if getattr(args, "tiled", False):
        return "tiled"
    if B <= 2 and has_qkv0_table(g):
        return "dataflow"
    if B <= 16 and has_qkv0_table(g) and g.weight_dtype == "bf16":
        return "flow"
    qd = g.n_q_heads * g.head_dim
    nqkv = (g.n_q_heads + 2 * g.n_kv_heads) * g.head_dim
    if (g.weight_dtype in ("bf16", "q8_0", "q4_0") and g.d_talker % 256 == 0 and g.d_model % 256 == 0 and g.d_model <= 4096 and g.d_talker <= 4096 and
            qd % 256 == 0 and g.d_ffn % 256 == 0 and nqkv % 32 == 0 and g.vocab % 32 == 0):
        return "tiled"
    return "generic"


TRAFFIC_FILES = {"dataflow": "k_stream", "flow": "k_flow", "tiled": "k_tiled"}


def measured_traffic(driver: str, workload: str):
    """HBM bytes per launch of a dataflow kernel (per frame call of the
    batched path: its staging copy, graph replay and output copy) from the
    committed counter summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain
    copy), or None when there is none for this driver and workload or the
    kernel's sources have changed since the counters were taken."""
    import hashlib
    if driver not in TRAFFIC_FILES:
        return None
    path = os.path.join(ROOT, "profiles", f"{TRAFFIC_FILES[driver]}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        kv[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in kv.get("sources", "").split():
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != kv.get("sources_sha256"):
        return None
    return int(kv["traffic_bytes_per_launch"])


def mfma_peak():
    """The measured dense bf16 matrix-core rate of this GPU (the probe in
    libqp_probe.so: back-to-back v_mfma_f32_16x16x32_bf16 in every wave of 4
    workgroups per compute unit), TFLOP/s, or None if the probe is missing."""
    import ctypes as C
    path = os.path.join(ROOT, "rvq_codebook_code_amd", "libqp_probe.so")
    if not os.path.exists(path):
        return None
    lib = C.CDLL(path)
    lib.qp_probe_mfma_bf16.argtypes = [C.c_int, C.c_int, C.c_int, C.POINTER(C.c_float), C.POINTER(C.c_double)]
    lib.qp_probe_mfma_bf16.restype = C.c_int
    ms, tf = C.c_float(), C.c_double()
    rc = lib.qp_probe_mfma_bf16(4, 20000, 5, C.byref(ms), C.byref(tf))
    if rc != 0:
        raise RuntimeError(f"matrix-core probe failed (HIP error {rc})")
    return round(tf.value, 1)


def exchange_probe():
    """Microseconds per tagged-record hand-off (libqp_probe.so): records per
    phase x consumer workgroups x waves per workgroup x loads in flight."""
    import ctypes as C
    lib = C.CDLL(os.path.join(ROOT, "rvq_codebook_code_amd", "libqp_probe.so"))
    lib.qp_probe_exchange.argtypes = [C.c_int] * 6 + [C.POINTER(C.c_float)]
    lib.qp_probe_exchange.restype = C.c_int
    out = []
    for waves, loads in ((4, 8), (4, 16), (8, 8), (16, 8)):
        for R in (1024, 4096, 8192, 16384, 32768, 49152):
            for consumers in (64, 256):
                us = C.c_float()
                rc = lib.qp_probe_exchange(R, consumers, waves, loads, 200, 3, C.byref(us))
                if rc == -1:
                    continue
                if rc != 0:
                    raise RuntimeError(f"exchange probe failed ({rc})")
                out.append({"records": R, "kib_per_consumer": R * 8 // 1024, "consumers": consumers,
                            "waves": waves, "loads_in_flight": loads, "us_per_phase": round(us.value, 3)})
                print(json.dumps(out[-1]), flush=True)
    return out


def boundary_probe():
    """Microseconds per kernel of back-to-back launches of a trivial kernel
    (libqp_probe.so): in one replayed graph or on a stream, with no work or
    writing / reading a buffer, over 200 launches of 256-thread workgroups."""
    import ctypes as C
    lib = C.CDLL(os.path.join(ROOT, "rvq_codebook_code_amd", "libqp_probe.so"))
    lib.qp_probe_boundary.argtypes = [C.c_int, C.c_int, C.c_size_t, C.c_int, C.c_int, C.c_int, C.POINTER(C.c_float)]
    lib.qp_probe_boundary.restype = C.c_int
    names = {0: "no work", 1: "writes", 2: "reads"}
    out = []
    cases = [(0, b, 0) for b in (256, 512, 1024)] + [(1, 512, n) for n in (1 << 16, 1 << 18, 1 << 20, 1 << 22)] + \
            [(2, 512, n) for n in (1 << 20, 1 << 23)]
    for graph in (1, 0):
        for kind, blocks, n in cases:
            us = C.c_float()
            rc = lib.qp_probe_boundary(kind, blocks, n, 200, graph, 5, C.byref(us))
            if rc != 0:
                raise RuntimeError(f"boundary probe failed ({rc})")
            out.append({"launch": "graph" if graph else "stream", "kernel": names[kind], "workgroups": blocks,
                        "kib": n * 4 // 1024, "us_per_kernel": round(us.value, 3)})
            print(json.dumps(out[-1]), flush=True)
    return out


def timeline(args, torch, dev):
    """Per-phase timeline of a dataflow frame kernel, from libqp_timeline.so
    (the same sources built with QP_TIMELINE: thread 0 of every workgroup
    writes the 100 MHz real-time counter at each phase's start, when its
    inputs are staged and at its end, into the taps buffer).  Four frames of
    the workload; the last is analysed over steps 2-15 (one position each).
    Per phase type: the hand-off (from the last workgroup to end the previous
    phase to the first one with its inputs staged), the median work (staged
    inputs to end), and the spread until the last workgroup ends."""
    import numpy as np
    from rvq_codebook_code_amd import binding as bd
    from rvq_codebook_code_amd import build as bb
    lib = bd.load_library(bb.TIMELINE_LIB)
    wl = synth.WORKLOADS[args.workload]
    g = wl.geom
    B = args.batch or wl.batch
    W = synth.make_weights(g, wl.weight_seed)
    pred = bd.Predictor(W, g, max_batch=B)
    H, q0 = synth.make_inputs(g, B, 4, wl.input_seed)
    if select_driver(g, B, args) == "tiled":
        return kernel_timeline(args, torch, dev, lib, pred, H, q0, B)
    nph = 400
    buf = torch.zeros(256 * nph * 3, dtype=torch.int64, device=dev)
    tok = torch.zeros((B, 15), dtype=torch.int32, device=dev)
    emb = torch.zeros((B, g.d_talker), dtype=torch.float32, device=dev)
    flags = bd.QP_FLAG_FLOW if args.flow else 0
    stream = torch.cuda.current_stream(dev).cuda_stream
    for f in range(4):
        buf.zero_()
        Hd = torch.from_numpy(H[f]).to(dev)
        qd = torch.from_numpy(q0[f]).to(dev)
        st = lib.qp_run_frames_ex(pred.h, B, Hd.data_ptr(), qd.data_ptr(), tok.data_ptr(), emb.data_ptr(), stream,
                                  None, None, buf.data_ptr(), flags)
        if st != 0:
            raise RuntimeError(f"qp_run_frames_ex failed ({st})")
        torch.cuda.synchronize()
    if pred.get_error() != 0:
        raise RuntimeError("device flags raised during the timeline frames")
    driver = "flow" if (args.flow or B >= 3) else "dataflow"
    pred.close()
    out = {"timeline": args.workload, "batch": B, "driver": driver}
    out.update(analyze_timeline(buf.cpu().numpy().reshape(256, nph, 3), g.n_layers))
    print(json.dumps(out), flush=True)


TL_NAMES = {1: "proj", 2: "qkv", 3: "attn", 4: "attn_tok", 5: "o", 6: "swiglu", 7: "down", 8: "lm", 9: "start",
            10: "next"}
TL_LAUNCHES, TL_WGS = 448, 1024


def kernel_timeline(args, torch, dev, lib, pred, H, q0, B):
    """Kernel timeline of the batched path (libqp_timeline.so): four frames
    through the prepared graph, as the bench runs them; thread 0 of every
    workgroup stamps each kernel's start, the end of a product's K loop (or
    an attention's staged inputs) and its end.  The last frame is summarised per kernel role."""
    import ctypes as C
    import numpy as np
    g = pred.geom
    tok = torch.zeros((B, 15), dtype=torch.int32, device=dev)
    emb = torch.zeros((B, g.d_talker), dtype=torch.float32, device=dev)
    for f in range(4):
        pred.run(torch.from_numpy(H[f]).to(dev), torch.from_numpy(q0[f]).to(dev), tok, emb, tiled=args.tiled)
    torch.cuda.synchronize()
    if pred.get_error() != 0:
        raise RuntimeError("device flags raised during the timeline frames")
    stamps = np.zeros(TL_LAUNCHES * TL_WGS * 3, dtype=np.uint64)
    kinds = (C.c_int * TL_LAUNCHES)()
    lib.qp_timeline_tiled.argtypes = [C.c_void_p, C.c_size_t, C.POINTER(C.c_int), C.c_int]
    lib.qp_timeline_tiled.restype = C.c_int
    n = lib.qp_timeline_tiled(stamps.ctypes.data, stamps.nbytes, kinds, TL_LAUNCHES)
    if n < 0:
        raise RuntimeError("qp_timeline_tiled failed")
    pred.close()
    out = {"timeline": args.workload, "batch": B, "driver": "tiled"}
    out.update(analyze_kernel_timeline(stamps.reshape(TL_LAUNCHES, TL_WGS, 3)[:n], list(kinds)[:n]))
    print(json.dumps(out), flush=True)


def analyze_kernel_timeline(stamps, kinds) -> dict:
    """Per-role statistics of one frame's kernel stamps [launches][workgroups][3]
    (raw 100 MHz counter values; k = 0 start, 1 end of a product's K loop or
    an attention's staged inputs (k1), 2 end; 0 where no workgroup wrote).  A
    launch's span runs from its first workgroup's start to its last one's end,
    its gap from the previous launch's last end to its first start.
    Workgroups that started before the frame's first launch (left from an
    earlier frame of another shape) are ignored."""
    import numpy as np
    T = stamps.astype(np.float64)
    first = T[0, :, 0]
    t0 = first[first > 0].min()
    per = {}
    prev_end = None
    tot_span = tot_gap = 0.0
    for i in range(T.shape[0]):
        w = T[i][(T[i, :, 0] >= t0) & (T[i, :, 2] > 0)]
        if len(w) == 0:
            continue
        start, end = w[:, 0].min(), w[:, 2].max()
        rec = per.setdefault(TL_NAMES.get(kinds[i], str(kinds[i])), {"span": [], "gap": [], "ramp": [], "wg": [],
                                                                      "loop": []})
        rec["span"].append((end - start) / 100.0)
        rec["ramp"].append((w[:, 0].max() - start) / 100.0)
        rec["wg"].append(float(np.median(w[:, 2] - w[:, 0])) / 100.0)
        if (w[:, 1] > 0).all():
            rec["loop"].append(float(np.median(w[:, 1] - w[:, 0])) / 100.0)
        tot_span += (end - start) / 100.0
        if prev_end is not None:
            rec["gap"].append((start - prev_end) / 100.0)
            tot_gap += (start - prev_end) / 100.0
        prev_end = end
    frame = (prev_end - t0) / 100.0
    out = {"frame_span_us": round(frame, 1), "kernels": int(sum(len(r["span"]) for r in per.values())),
           "kernel_time_us": round(tot_span, 1), "gap_time_us": round(tot_gap, 1), "per_kernel_us": {}}
    for k, r in per.items():
        m = lambda v: round(float(np.mean(v)), 2) if v else None
        out["per_kernel_us"][k] = {"launches": len(r["span"]), "span": m(r["span"]), "gap_before": m(r["gap"]),
                                   "start_ramp": m(r["ramp"]), "workgroup_median": m(r["wg"]),
                                   "k1_median": m(r["loop"]), "total": round(float(np.sum(r["span"])), 1)}
    return out


def analyze_timeline(stamps, L: int) -> dict:
    """Per-phase-type statistics of one frame's stamps [workgroups][phases][3]
    (raw 100 MHz counter values, 0 where a workgroup took no part): phase ph
    of step s, layer l, type t is 1 + (s - 1) (5 L + 1) + 5 l + t, the lm_head
    of step s 1 + (s - 1) (5 L + 1) + 5 L.  Steps 2-15 are averaged."""
    import numpy as np
    T = stamps.astype(np.float64)
    nph = T.shape[1]
    have = T[:, :, 0] > 0
    t_first = T[have].min()
    T = np.where(T > 0, (T - t_first) / 100.0, np.nan)          # microseconds
    names = ["qkv", "attn", "o", "up", "down"]
    per = {n: [] for n in names + ["lm"]}
    prev_end = None
    span_phases = 0
    for ph in range(1, nph):
        w = np.where(have[:, ph])[0]
        if len(w) == 0:
            continue
        span_phases += 1
        q = (ph - 1) % (5 * L + 1)
        s = 1 + (ph - 1) // (5 * L + 1)
        kind = "lm" if q == 5 * L else names[q % 5]
        ready = np.nanmin(T[w, ph, 1])
        end_last = np.nanmax(T[w, ph, 2])
        if s >= 2 and prev_end is not None:
            per[kind].append([ready - prev_end, np.nanmedian(T[w, ph, 2] - T[w, ph, 1]),
                              end_last - np.nanmin(T[w, ph, 2]), end_last - ready])
        prev_end = end_last
    span = np.nanmax(T[:, :, 2]) - np.nanmin(T[:, :, 0])
    out = {"frame_span_us": round(float(span), 1), "phases_with_exchange": span_phases,
           "us_per_phase": round(float(span) / max(span_phases, 1), 3), "per_phase_type_us": {}}
    for k, v in per.items():
        if not v:
            continue
        a = np.nanmean(np.array(v), axis=0)
        out["per_phase_type_us"][k] = {"handoff": round(float(a[0]), 2), "work_median": round(float(a[1]), 2),
                                       "end_spread": round(float(a[2]), 2), "ready_to_last_end": round(float(a[3]), 2),
                                       "phases": len(v)}
    return out


def batch_mix(args, torch, dev):
    """Frames whose batch size changes from call to call, enqueued back to back
    with no synchronisation (as a scheduler that fills each frame with the
    requests at hand would), against the same frames at a fixed batch: the
    handle's prepared graphs serve every batch size without capture or
    allocation, so a changing B costs only the size of its bucket."""
    from rvq_codebook_code_amd import binding as bd
    wl = synth.WORKLOADS[args.workload]
    g = wl.geom
    sizes = [int(x) for x in args.batch_mix.split(",")]
    Bmax = max(sizes)
    W = synth.make_weights(g, wl.weight_seed)
    H, q0 = synth.make_inputs(g, Bmax, 4, wl.input_seed)
    pred = bd.Predictor(W, g, max_batch=Bmax)
    Hd = torch.from_numpy(H).to(dev)
    qd = torch.from_numpy(q0).to(dev)
    tok = torch.zeros((Bmax, 15), dtype=torch.int32, device=dev)
    emb = torch.zeros((Bmax, g.d_talker), dtype=torch.float32, device=dev)

    def run(seq):
        for i, B in enumerate(seq):
            pred.run(Hd[i % 4, :B], qd[i % 4, :B], tok[:B], emb[:B])

    def timed(seq):
        run(seq[:len(sizes)])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(seq)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3
    reps = max(1, args.steps // len(sizes))
    mixed = sizes * reps
    ms_mixed = timed(mixed)
    fixed = {}
    for B in sorted(set(sizes)):
        fixed[B] = timed([B] * reps) / reps
    ms_sum_fixed = sum(fixed[B] for B in sizes) * reps
    if pred.get_error() != 0:
        raise RuntimeError("device flags raised during the batch mix")
    pred.close()
    print(json.dumps({"batch_mix": sizes, "workload": args.workload, "calls": len(mixed),
                      "ms_mixed_sequence": round(ms_mixed, 3),
                      "ms_same_calls_each_size_alone": round(ms_sum_fixed, 3),
                      "ms_per_call_by_size": {str(B): round(v, 4) for B, v in fixed.items()},
                      "frames_per_s_mixed": round(sum(mixed) / ms_mixed * 1e3, 1)}), flush=True)


LIBRARY_GEMM_SHAPES = ("qkv", "o", "gateup", "down")


def library_gemm(args, torch, dev):
    """The vendor library (torch.mm, hipBLASLt on this image) on one of the
    1.7B-shaped predictor's bf16 products, [B x K] . [K x N], in the regime the
    batched path's frames run in: 100 products captured in one graph and
    replayed back to back.  Shapes: q/k/v [1024 x 4096], output projection
    [2048 x 1024], gate and up as one [1024 x 6144] product, down
    [3072 x 1024].  Eight weight copies are used in turn (64-96 MiB, more than
    the L2s hold).  The JSON line gives the time per product over 20 replays
    (kernel and the gap before the next one); the outputs are not used."""
    shapes = {"qkv": (1024, 4096), "o": (2048, 1024), "gateup": (1024, 6144), "down": (3072, 1024)}
    K, N = shapes[args.library_gemm]
    M = args.batch or 128
    gen = torch.Generator(device=dev).manual_seed(7)
    A = torch.randn(M, K, device=dev, dtype=torch.bfloat16, generator=gen)
    Ws = [torch.randn(K, N, device=dev, dtype=torch.bfloat16, generator=gen) for _ in range(8)]
    out = torch.empty(M, N, device=dev, dtype=torch.bfloat16)
    per_graph = 100
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for i in range(20):
            torch.mm(A, Ws[i % 8], out=out)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(per_graph):
            torch.mm(A, Ws[i % 8], out=out)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    reps = 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * per_graph)
    print(json.dumps({"library_gemm": args.library_gemm, "M": M, "K": K, "N": N, "products_per_graph": per_graph,
                      "replays": reps, "us_per_product_in_graph": round(us, 3),
                      "tflops": round(2.0 * M * K * N / us / 1e6, 2)}), flush=True)


def calibrate_copy(torch, dev):
    """A plain copy of COPY_BYTES, five times: the reference for scaling the
    FETCH_SIZE / WRITE_SIZE counters (each launch reads and writes exactly
    COPY_BYTES)."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": COPY_BYTES, "launches": 5}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="b1", choices=sorted(synth.WORKLOADS) + sorted(synth.TALKER_WORKLOADS))
    ap.add_argument("--stepwise", action="store_true", help="one kernel per phase instead of the persistent kernel")
    ap.add_argument("--generic", action="store_true", help="the generic persistent kernel even where a specialised one exists")
    ap.add_argument("--flow", action="store_true",
                    help="the moderate-batch dataflow kernel at any B <= 16 (1.7B geometry, bf16 weights)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sample", default=None, metavar="T,K,P",
                    help="draw every token (temperature T, top-k K, top-p P) with seeded uniforms instead of the argmax")
    ap.add_argument("--batch", type=int, default=None,
                    help="run the workload's weights at this batch size instead of its own (crossover sweeps)")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="before every timed frame copy this many MiB (evicting the MALL); the frame alone is timed")
    ap.add_argument("--mfma-peak", action="store_true", help="only run the matrix-core peak probe")
    ap.add_argument("--exchange-probe", action="store_true", help="only run the tagged-record hand-off probe")
    ap.add_argument("--boundary-probe", action="store_true", help="only run the kernel-boundary probe")
    ap.add_argument("--batch-mix", default=None,
                    help="comma-separated batch sizes cycled call by call (e.g. 1,3,16,40,128)")
    ap.add_argument("--timeline", action="store_true",
                    help="per-phase timeline of the workload's dataflow kernel, or the kernel timeline of "
                         "the batched path (libqp_timeline.so)")
    ap.add_argument("--tiled", action="store_true", help="the batched matrix-core path at any B")
    ap.add_argument("--library-gemm", choices=LIBRARY_GEMM_SHAPES,
                    help="torch.mm (the vendor library) on one of the predictor's product shapes at --batch rows")
    ap.add_argument("--only", action="store_true",
                    help="time the named workload alone (by default the b1 line also times b16 and b128)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of known size (to scale HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(requests shard by replication, see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from rvq_codebook_code_amd import binding as bd

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        calibrate_copy(torch, dev)
        return
    if args.exchange_probe:
        exchange_probe()
        return
    if args.boundary_probe:
        boundary_probe()
        return
    if args.timeline:
        timeline(args, torch, dev)
        return
    if args.library_gemm:
        library_gemm(args, torch, dev)
        return
    if args.batch_mix:
        batch_mix(args, torch, dev)
        return
    if args.mfma_peak:
        print(json.dumps({"mfma_peak_bf16_tflops": mfma_peak(), "vendor_dense_bf16_tflops": MFMA_BF16_PEAK_TFLOPS}),
              flush=True)
        return
    if args.workload in synth.TALKER_WORKLOADS:
        run_talker(args, torch, dev)
        return
    line = measure(args.workload, args, torch, dev, bd)
    if (args.workload == "b1" and not args.only and not args.sample
            and not (args.stepwise or args.generic or args.flow or args.tiled)
            and args.batch is None and not args.flush_mib):
        # the metric is quoted at B = 1, 16 and 128: the other two batch sizes
        # are timed in the same run, each with its own roofline and oracle
        line["workloads"] = {}
        for name in ("b16", "b128"):
            sub = measure(name, args, torch, dev, bd)
            line["workloads"][name] = {k: sub[k] for k in ("value", "unit", "ms_per_step", "dtype", "config",
                                                           "roofline", "cpu_baseline", "free_run_vs_oracle")}
        # the B = 128 line is graded on the matrix cores: also against this
        # GPU's measured peak of the instruction the products use
        peak = mfma_peak()
        if peak:
            rf = line["workloads"]["b128"]["roofline"]
            rf["peak_measured"] = peak
            rf["frac_of_measured_peak"] = round(rf["achieved"] / peak, 4)
    print(json.dumps(line), flush=True)


def measure(name, args, torch, dev, bd):
    """Time one workload (frames of its batch, inputs resident on the GPU) and
    return its JSON record."""
    wl = synth.WORKLOADS[name]
    g = wl.geom
    B = wl.batch if args.batch is None else args.batch
    W = synth.make_weights(g, wl.weight_seed)
    H, q0 = synth.make_inputs(g, B, wl.frames, wl.input_seed)
    pred = bd.Predictor(W, g, max_batch=B)
    Hd = torch.from_numpy(H).to(dev)
    qd = torch.from_numpy(q0).to(dev)
    tok = torch.zeros((B, 15), dtype=torch.int32, device=dev)
    emb = torch.zeros((B, g.d_talker), dtype=torch.float32, device=dev)
    F = H.shape[0]
    sampling = None
    if args.sample:
        t_, k_, p_ = args.sample.split(",")
        sampling = (float(t_), int(k_), float(p_))
        U = synth.make_uniforms(B, F, wl.input_seed + 7)
        Ud = torch.from_numpy(U).to(dev)

    def frame(i):
        if sampling is None:
            pred.run(Hd[i % F], qd[i % F], tok, emb, stepwise=args.stepwise, generic=args.generic,
                     flow=args.flow, tiled=args.tiled)
        else:
            pred.run_sampled(Hd[i % F], qd[i % F], Ud[i % F], tok, emb, *sampling)

    for i in range(args.warmup):
        frame(i)
    torch.cuda.synchronize()
    if pred.get_error() != 0:
        raise RuntimeError("device flag raised during warm-up")

    stream = torch.cuda.current_stream(dev)
    # one event pair per frame call, on the stream the library launches on:
    # for the single-kernel drivers that brackets exactly one kernel launch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    flush = None
    if args.flush_mib:
        flush = (torch.empty(args.flush_mib << 18, dtype=torch.float32, device=dev).uniform_(),
                 torch.empty(args.flush_mib << 18, dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    for i in range(args.steps):
        if flush is not None:
            flush[1].copy_(flush[0])      # evicts the frame's weights from the MALL
        ev[i][0].record(stream)
        frame(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0][0].elapsed_time(ev[-1][1])
    launch_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    if pred.get_error() != 0:
        raise RuntimeError("device flag raised during the timed frames")
    if flush is not None:
        # the copies sit between the frames: only the frames are timed
        ms = launch_ms * args.steps
    ms_per_step = ms / args.steps
    frames_per_s = B * args.steps / (ms / 1e3)

    driver = select_driver(g, B, args)
    # the dataflow and batched drivers read layer 0's q/k/v rows of steps
    # 2..15 from the create-time table
    table = driver in ("dataflow", "flow", "tiled") and has_qkv0_table(g)
    nbytes = algorithmic_bytes(g, B, qkv0_table=table)
    nflops = algorithmic_flops(g, B, qkv0_table=table)
    # the unreduced models: every step streams layer 0's q/k/v weights too;
    # the flops of the whole frame, the prefill's second row and attention included
    nbytes_full = algorithmic_bytes(g, B, qkv0_table=False)
    nflops_full = model_flops(g, B)
    # achieved: per call, over the mean event-pair duration around each call
    # (the dataflow driver: exactly one kernel launch; the batched driver: the
    # staging copies and the graph replay of the frame's kernels); the
    # end-to-end fraction uses ms_per_step, gaps between calls included
    scope = "one kernel launch" if driver in ("dataflow", "flow", "generic") else "one frame call (staging + graph replay)"
    if B >= 128:
        # throughput batch: graded against the bf16 matrix-core peak
        achieved = nflops / (launch_ms / 1e3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": (measured_traffic(driver, wl.name)
                                if B == wl.batch and not args.flush_mib else None),
                    "frac_end_to_end": round(nflops / (ms_per_step / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                    "frac_unreduced_model": round(nflops_full / (launch_ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                    "algorithmic_flops_unreduced": nflops_full, "per": scope}
    else:
        achieved_gbs = nbytes / (launch_ms / 1e3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                    "traffic": (measured_traffic(driver, wl.name)
                                if B == wl.batch and not args.flush_mib else None),
                    "frac_end_to_end": round(nbytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                    "frac_unreduced_model": round(nbytes_full / (launch_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                    "algorithmic_bytes_unreduced": nbytes_full, "per": scope}

    cpu = None
    free_run = None
    if not args.no_cpu_baseline:
        cpu, outs = cpu_baseline(wl, W, H, q0, args.cpu_budget, sampling, U if sampling else None)
        # the same frames again on the GPU, untimed, for their tokens
        got = []
        for i in range(len(outs)):
            frame(i)
            got.append(tok.cpu().numpy().copy())
        free_run = free_run_agreement(got, outs)

    # arithmetic type of the products: bf16 operands with fp32 accumulation
    # on the matrix cores and in the dataflow kernel with bf16 weights; the
    # dataflow kernel multiplies Q8_0 / Q4_0 codes with fp32 activations, and
    # the generic path computes in fp32
    if driver in ("tiled", "flow") or (driver == "dataflow" and g.weight_dtype == "bf16"):
        dtype = "bf16"
    else:
        dtype = "f32"
    line = {
        "metric": METRIC,
        "value": round(frames_per_s, 2),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": wl.name if args.batch is None else f"{wl.name} weights at B={B}", "batch": B,
                   "frames_per_step": 1, "mall_flush_mib_before_each_frame": args.flush_mib or None,
                   "weights": g.weight_dtype, "embeddings": g.emb_format,
                   "predictor": f"dP={g.d_model} L={g.n_layers} heads={g.n_q_heads}/{g.n_kv_heads}x{g.head_dim} "
                                f"F={g.d_ffn} V={g.vocab} dT={g.d_talker}",
                   "driver": driver,
                   "sampling": (None if sampling is None else
                                {"temperature": sampling[0], "top_k": sampling[1], "top_p": sampling[2],
                                 "uniforms": "seeded, one per request and step"}),
                   "ms_per_launch": round(launch_ms, 4),
                   "tokens_per_s": round(15 * frames_per_s, 1),
                   "algorithmic_bytes_per_step": nbytes,
                   "algorithmic_flops_per_step": nflops},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "free_run_vs_oracle": free_run,
    }
    # every launch has finished before the handle is destroyed
    torch.cuda.synchronize()
    pred.close()
    return line


if __name__ == "__main__":
    main()
