"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

Bar (per workload): under teacher forcing with the oracle's own tokens,
  * tokens equal wherever the oracle's top-2 logit margin exceeds 0.05,
  * at every step (decisive or not) the GPU's token is the lowest-index
    argmax of its own fp32 logits, and the oracle's logit at that token lies
    within twice the measured logit error of the oracle's maximum (what any
    correct argmax of logits that close must satisfy),
  * logits and embsum within max-abs 1e-4 for fp32 weights, 3e-2 for bf16
    and Q8_0 weights.
Free-run token agreement is printed as context.  The 1.7B-shaped workloads
run on handles built as the bench builds them (max_batch = the workload's
batch) and compare every row of whole frames.
"""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import predictor as O
from rvq_codebook_code_amd import binding as bd
from rvq_codebook_code_amd import synth

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 3e-2, "q8_0": 3e-2, "q4_0": 3e-2}
MARGIN = 0.05


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


_cache = {}


def workload(name):
    """(workload, weights, oracle model, predictor) built once per session."""
    _dev()
    if name not in _cache:
        wl = synth.WORKLOADS[name]
        W = synth.make_weights(wl.geom, wl.weight_seed)
        model = O.OracleModel(W, wl.geom)
        pred = bd.Predictor(W, wl.geom, max_batch=max(wl.batch, 40))
        _cache[name] = (wl, W, model, pred)
    return _cache[name]


def gpu_frame(pred, H, q0, force=None, logits=True, taps=False, stepwise=False, generic=False, tiled=False,
              flow=False):
    dev = _dev()
    g = pred.geom
    B = H.shape[0]
    Ht = torch.from_numpy(np.ascontiguousarray(H, dtype=np.float32)).to(dev)
    qt = torch.from_numpy(np.ascontiguousarray(q0, dtype=np.int32)).to(dev)
    tok = torch.full((B, 15), -1, dtype=torch.int32, device=dev)
    emb = torch.full((B, g.d_talker), float("nan"), dtype=torch.float32, device=dev)
    ft = None if force is None else torch.from_numpy(np.ascontiguousarray(force, dtype=np.int32)).to(dev)
    lg = torch.full((B, 15, g.vocab), float("nan"), dtype=torch.float32, device=dev) if logits else None
    tp = (torch.full((16, g.n_layers, B, g.d_model), float("nan"), dtype=torch.float32, device=dev)
          if taps else None)
    pred.run(Ht, qt, tok, emb, force=ft, logits_out=lg, taps_out=tp, stepwise=stepwise, generic=generic,
             tiled=tiled, flow=flow)
    torch.cuda.synchronize()
    assert pred.get_error() == 0
    out = {"tokens": tok.cpu().numpy(), "embsum": emb.cpu().numpy()}
    if logits:
        out["logits"] = lg.cpu().numpy()
    if taps:
        out["taps"] = tp.cpu().numpy()
    return out


def check_against_oracle(name, model, pred, H, q0, rows, stepwise=False, tiled=False, flow=False):
    """Teacher-forced comparison of the sampled ``rows`` of one frame."""
    tol = TOL[model.g.weight_dtype]
    ref = O.run_frames(model, H[rows], q0[rows])
    force = np.zeros((H.shape[0], 15), dtype=np.int32)
    force[rows] = ref["tokens"]
    got = gpu_frame(pred, H, q0, force=force, stepwise=stepwise, tiled=tiled, flow=flow)
    lg_err = np.abs(got["logits"][rows] - ref["logits"]).max()
    em_err = np.abs(got["embsum"][rows] - ref["embsum"]).max()
    sure = ref["margin"] > MARGIN
    gtok = got["tokens"][rows]
    tok_ok = (gtok == ref["tokens"])
    print(f"[{name}] rows={len(rows)} logits max-abs {lg_err:.3g} embsum max-abs {em_err:.3g} "
          f"decisive {sure.mean():.2f} token agreement {tok_ok.mean():.3f}")
    assert np.isfinite(got["logits"][rows]).all()
    assert lg_err <= tol
    assert em_err <= tol
    assert tok_ok[sure].all()
    check_every_step(got["logits"][rows], gtok, ref["logits"], lg_err)
    return ref, got


def check_every_step(glog, gtok, rlog, lg_err):
    """Every step, decisive or not: the GPU's token is the lowest-index argmax
    of its own fp32 logits (exact), and the oracle's logit at that token is
    within 2 * lg_err (+ fp32 rounding) of the oracle's largest logit; with
    |gpu - oracle| <= lg_err everywhere, an argmax of the GPU's logits can be
    no further below the oracle's maximum."""
    own = np.argmax(glog.astype(np.float32), axis=-1)
    np.testing.assert_array_equal(gtok, own)
    at_tok = np.take_along_axis(rlog, gtok[..., None].astype(np.int64), axis=-1)[..., 0]
    short = rlog.max(axis=-1) - at_tok
    assert (short <= 2.0 * lg_err + 1e-6).all(), float(short.max())


# ----------------------------------------------------------------------------
# tiny fp32 workload: every frame, both drivers, per-layer taps
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("stepwise", [False, True], ids=["persistent", "stepwise"])
def test_tiny_all_frames(stepwise):
    wl, W, model, pred = workload("tiny")
    H, q0 = synth.make_inputs(wl.geom, wl.batch, wl.frames, wl.input_seed)
    rows = np.arange(wl.batch)
    for f in range(wl.frames):
        check_against_oracle("tiny", model, pred, H[f], q0[f], rows, stepwise=stepwise)


def test_tiny_free_run_and_taps():
    wl, W, model, pred = workload("tiny")
    H, q0 = synth.make_inputs(wl.geom, wl.batch, 2, wl.input_seed + 1)
    ref = O.run_frames(model, H[0], q0[0], want_taps=True)
    got = gpu_frame(pred, H[0], q0[0], taps=True)
    np.testing.assert_allclose(got["taps"], ref["taps"], atol=1e-4, rtol=0)
    # free run: the decisive prefix must agree token for token
    for b in range(wl.batch):
        for k in range(15):
            if ref["margin"][b, k] <= MARGIN:
                break
            assert got["tokens"][b, k] == ref["tokens"][b, k]
    # greedy consistency on the GPU: re-forcing its own tokens changes nothing
    again = gpu_frame(pred, H[0], q0[0], force=got["tokens"])
    np.testing.assert_array_equal(again["tokens"], got["tokens"])
    np.testing.assert_array_equal(again["logits"], got["logits"])
    np.testing.assert_array_equal(again["embsum"], got["embsum"])


def test_tiny_batch_composition_and_determinism():
    wl, W, model, pred = workload("tiny")
    H, q0 = synth.make_inputs(wl.geom, 8, 1, 77)
    full = gpu_frame(pred, H[0], q0[0])
    perm = np.array([5, 1, 7])
    sub = gpu_frame(pred, H[0][perm], q0[0][perm])
    for key in ("tokens", "logits", "embsum"):
        np.testing.assert_array_equal(sub[key], full[key][perm])
    one = gpu_frame(pred, H[0][3:4], q0[0][3:4], stepwise=True)
    for key in ("tokens", "logits", "embsum"):
        np.testing.assert_array_equal(one[key], full[key][3:4])
    for _ in range(3):
        rep = gpu_frame(pred, H[0], q0[0])
        for key in ("tokens", "logits", "embsum"):
            np.testing.assert_array_equal(rep[key], full[key])


def test_edge_cases_and_flags():
    wl, W, model, pred = workload("tiny")
    dev = _dev()
    g = wl.geom
    # B = 0 is a no-op
    z = torch.zeros((0, g.d_talker), dtype=torch.float32, device=dev)
    pred.run(z, torch.zeros((0,), dtype=torch.int32, device=dev),
             torch.zeros((0, 15), dtype=torch.int32, device=dev), z.clone())
    # B above max_batch is refused on the host
    Bbig = pred.max_batch + 1
    with pytest.raises(bd.QpError) as ei:
        pred.run(torch.zeros((Bbig, g.d_talker), device=dev), torch.zeros((Bbig,), dtype=torch.int32, device=dev),
                 torch.zeros((Bbig, 15), dtype=torch.int32, device=dev),
                 torch.zeros((Bbig, g.d_talker), device=dev))
    assert ei.value.status == bd.QP_ERR_BATCH
    # an out-of-range q0 raises the sticky flag and is read as token 0
    H, q0 = synth.make_inputs(g, 2, 1, 5)
    bad = q0[0].copy()
    bad[1] = g.vocab + 3
    Ht = torch.from_numpy(H[0]).to(dev)
    tok = torch.zeros((2, 15), dtype=torch.int32, device=dev)
    emb = torch.zeros((2, g.d_talker), device=dev)
    pred.run(Ht, torch.from_numpy(bad).to(dev), tok, emb)
    torch.cuda.synchronize()
    assert pred.get_error() == 1
    assert pred.get_error() == 0
    fixed = bad.copy()
    fixed[1] = 0
    ref = gpu_frame(pred, H[0], fixed)
    np.testing.assert_array_equal(tok.cpu().numpy(), ref["tokens"])
    # the batched matrix-core path takes bf16 / Q8_0 weights only, alone
    with pytest.raises(bd.QpError) as ei:
        gpu_frame(pred, H[0], q0[0], tiled=True)
    assert ei.value.status == bd.QP_ERR_INVALID_ARG
    _, _, _, pb = workload("tiny_bf16")
    with pytest.raises(bd.QpError) as ei:
        gpu_frame(pb, H[0], q0[0], tiled=True, generic=True)
    assert ei.value.status == bd.QP_ERR_INVALID_ARG


# ----------------------------------------------------------------------------
# 1.7B-shaped workloads at their full batch sizes, sampled rows
# ----------------------------------------------------------------------------

def bench_handle(name):
    """The workload's predictor built as bench.py builds it: max_batch equal to
    the workload's batch (the KV-cache and scratch strides of the timed
    configuration)."""
    wl, W, model, _ = workload(name)
    key = "bench:" + name
    if key not in _cache:
        _cache[key] = bd.Predictor(W, wl.geom, max_batch=wl.batch)
    return wl, W, model, _cache[key]


@pytest.mark.parametrize("name,frames", [
    ("b1", [0, 1, 255]),
    ("b16", [0, 127]),
    ("b128", [0, 63]),
    ("q8ema", [0, 63]),
])
def test_full_size_whole_frames(name, frames):
    """Every row of whole frames of the 1.7B-shaped workloads, in the bench's
    launch configuration, against the oracle under teacher forcing; then the
    same frames free-running (no hooks: the launch the bench times), their
    token agreement with the oracle's free run printed as context and the
    tokens up to each row's first non-decisive step required equal."""
    wl, W, model, pred = bench_handle(name)
    H, q0 = synth.make_inputs(wl.geom, wl.batch, wl.frames, wl.input_seed)
    rows = np.arange(wl.batch)
    for f in frames:
        ref, _ = check_against_oracle(f"{name} frame {f}", model, pred, H[f], q0[f], rows)
        free = gpu_frame(pred, H[f], q0[f], logits=False)
        agree = (free["tokens"] == ref["tokens"])
        prefix = np.cumprod(agree, axis=1).sum(axis=1)
        first_open = np.argmax(np.concatenate([ref["margin"] <= MARGIN, np.ones((len(rows), 1), bool)], axis=1),
                               axis=1)
        print(f"[{name} frame {f} free run] token agreement {agree.mean():.3f}, "
              f"mean agreeing prefix {prefix.mean():.2f} of 15")
        assert (prefix >= first_open).all()


# ----------------------------------------------------------------------------
# the small-batch dataflow kernel (1.7B geometry, bf16, B <= 2)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["b16", "q8ema", "q4_b16"])
@pytest.mark.parametrize("B", [1, 2])
def test_dataflow_kernel_against_oracle_and_generic(B, name):
    """bf16 weights, and Q8_0 / Q4_0 codes with their block scales (Q8_0
    with the EMA codebook tables)."""
    wl, W, model, pred = workload(name)
    H, q0 = synth.make_inputs(wl.geom, B, 3, 4242 + B)
    rows = np.arange(B)
    for f in range(3):
        ref, got = check_against_oracle(f"dataflow {name} B={B}", model, pred, H[f], q0[f], rows)
        force = ref["tokens"].astype(np.int32)
        # the dataflow kernel rounds its product operands to bf16 (the generic
        # path keeps them fp32): the two agree to the bf16-weight bar
        gen = gpu_frame(pred, H[f], q0[f], force=force, generic=True)
        lg = np.abs(gen["logits"] - got["logits"]).max()
        print(f"[dataflow {name} B={B} vs generic] logits max-abs {lg:.3g}")
        assert lg <= TOL["bf16"]
        assert np.abs(gen["embsum"] - got["embsum"]).max() <= 1e-5


def test_dataflow_record_tags_restart(monkeypatch):
    """The dataflow kernel's 32-bit record tags restart, after every record
    is cleared, before they would wrap (after about 11 million frames).  A
    handle that starts just below that point runs frames on both sides of the
    restart; they equal a fresh handle's bit for bit."""
    wl, W, model, pred = workload("b1")
    ppf = 1 + 15 * (5 * wl.geom.n_layers + 1) + 1
    last = 2**32 - 1 - 2 * ppf            # the highest start the kernel runs without a restart
    for start in (last - 100, last):
        monkeypatch.setenv("QP_TEST_EPOCH0", str(start))
        late = bd.Predictor(W, wl.geom, max_batch=2)
        monkeypatch.delenv("QP_TEST_EPOCH0")
        H, q0 = synth.make_inputs(wl.geom, 2, 3, 5150 + start % 7)
        for f in range(3):
            for B in (1, 2):
                a = gpu_frame(pred, H[f][:B], q0[f][:B])
                b = gpu_frame(late, H[f][:B], q0[f][:B])
                for key in ("tokens", "logits", "embsum"):
                    np.testing.assert_array_equal(a[key], b[key])
        late.close()


@pytest.mark.parametrize("name", ["b16", "q4_b16"])
def test_dataflow_table_rows_at_vocabulary_ends(name):
    """Forced tokens 0 and V-1 alternating (and q0 at both ends): the fed
    rows of the projected tables and of the layer-0 q/k/v table at the
    vocabulary's first and last index, on the dataflow kernel (B = 1, 2)
    against the oracle under the same forcing."""
    wl, W, model, pred = workload(name)
    V = wl.geom.vocab
    H, _ = synth.make_inputs(wl.geom, 2, 1, 8080)
    q0 = np.array([V - 1, 0], dtype=np.int32)
    force = np.zeros((2, 15), dtype=np.int32)
    force[0, 1::2] = V - 1
    force[1, 0::2] = V - 1
    for B in (1, 2):
        ref = O.run_frames(model, H[0][:B], q0[:B], force=force[:B])
        got = gpu_frame(pred, H[0][:B], q0[:B], force=force[:B])
        lg = np.abs(got["logits"] - ref["logits"]).max()
        em = np.abs(got["embsum"] - ref["embsum"]).max()
        print(f"[dataflow {name} ends B={B}] logits max-abs {lg:.3g} embsum max-abs {em:.3g}")
        assert lg <= TOL[wl.geom.weight_dtype] and em <= TOL[wl.geom.weight_dtype]
        sure = ref["margin"] > MARGIN
        assert (got["tokens"] == ref["tokens"])[sure].all()


@pytest.mark.parametrize("n_layers", [1, 2])
def test_dataflow_kernel_fewer_layers(n_layers):
    """The dataflow kernel takes 1 to 5 layers of the 1.7B widths: its phase
    count and weight-prefetch chain change with L (with one layer, layer 0 is
    also the last, and its q/k/v comes from the table from step 2 on).
    B = 1 and 2 against the oracle."""
    wl = synth.WORKLOADS["b16"]
    g = dataclasses.replace(wl.geom, n_layers=n_layers)
    W = synth.make_weights(g, wl.weight_seed)
    model = O.OracleModel(W, g)
    pred = bd.Predictor(W, g, max_batch=2)
    H, q0 = synth.make_inputs(g, 2, 2, 7070 + n_layers)
    for f in range(2):
        for B in (1, 2):
            check_against_oracle(f"dataflow L={n_layers} B={B}", model, pred, H[f][:B], q0[f][:B], np.arange(B))
    pred.close()


def test_dataflow_kernel_taps_and_repeat():
    wl, W, model, pred = workload("b1")
    H, q0 = synth.make_inputs(wl.geom, 1, 2, 777)
    ref = O.run_frames(model, H[0], q0[0], want_taps=True)
    got = gpu_frame(pred, H[0], q0[0], force=ref["tokens"].astype(np.int32), taps=True)
    err = np.abs(got["taps"] - ref["taps"]).max()
    print(f"[dataflow taps] max-abs {err:.3g}")
    assert err <= TOL["bf16"]
    again = gpu_frame(pred, H[0], q0[0], force=ref["tokens"].astype(np.int32), taps=True)
    for key in ("tokens", "logits", "embsum", "taps"):
        np.testing.assert_array_equal(again[key], got[key])


# ----------------------------------------------------------------------------
# the moderate-batch dataflow kernel (1.7B geometry, bf16, 3 <= B <= 16)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("B", [3, 8, 9, 16])
def test_flow_kernel_against_oracle_and_batched(B):
    """Every row of two frames against the oracle (B = 9 and 16: the prefill's
    2B rows span two 16-row fragments), then the same frames on the batched
    matrix-core path: the two round the same operands to bf16 and agree to
    the bf16 bar."""
    wl, W, model, pred = workload("b16")
    H, q0 = synth.make_inputs(wl.geom, B, 2, 8100 + B)
    for f in range(2):
        ref, got = check_against_oracle(f"flow B={B}", model, pred, H[f], q0[f], np.arange(B))
        tiled = gpu_frame(pred, H[f], q0[f], force=ref["tokens"].astype(np.int32), tiled=True)
        lg = np.abs(tiled["logits"] - got["logits"]).max()
        print(f"[flow B={B} vs batched] logits max-abs {lg:.3g}")
        assert lg <= TOL["bf16"]
        assert np.abs(tiled["embsum"] - got["embsum"]).max() <= 1e-5


@pytest.mark.parametrize("B", [1, 2])
def test_flow_kernel_small_batches_by_flag(B):
    """The same kernel at B = 1 and 2 (QP_FLAG_FLOW; by default those run on
    the small-batch kernel): one unit per kv head of each request."""
    wl, W, model, pred = workload("b16")
    H, q0 = synth.make_inputs(wl.geom, B, 1, 8200 + B)
    check_against_oracle(f"flow B={B} (flag)", model, pred, H[0], q0[0], np.arange(B), flow=True)


def test_flow_kernel_taps_composition_and_repeat():
    """Per-layer residual taps against the oracle's; a row's results do not
    depend on the batch it runs in (a permuted subset of a B = 12 frame
    reproduces its rows bit for bit); repeats are bit for bit."""
    wl, W, model, pred = workload("b16")
    H, q0 = synth.make_inputs(wl.geom, 12, 1, 8300)
    ref = O.run_frames(model, H[0][:5], q0[0][:5], want_taps=True)
    got = gpu_frame(pred, H[0][:5], q0[0][:5], force=ref["tokens"].astype(np.int32), taps=True)
    err = np.abs(got["taps"] - ref["taps"]).max()
    print(f"[flow taps] max-abs {err:.3g}")
    assert err <= TOL["bf16"]
    full = gpu_frame(pred, H[0], q0[0])
    perm = np.array([11, 2, 7, 0])
    sub = gpu_frame(pred, H[0][perm], q0[0][perm])
    for key in ("tokens", "logits", "embsum"):
        np.testing.assert_array_equal(sub[key], full[key][perm])
    for _ in range(3):
        rep = gpu_frame(pred, H[0], q0[0])
        for key in ("tokens", "logits", "embsum"):
            np.testing.assert_array_equal(rep[key], full[key])


def test_flow_kernel_flags():
    """An out-of-range q0 and an out-of-range forced token raise the sticky
    flag and are read as token 0; the next call is clean."""
    wl, W, model, pred = workload("b16")
    dev = _dev()
    g = wl.geom
    B = 6
    H, q0 = synth.make_inputs(g, B, 1, 8400)
    bad = q0[0].copy()
    bad[4] = g.vocab + 7
    fixed = bad.copy()
    fixed[4] = 0
    ref = gpu_frame(pred, H[0], fixed, logits=False)
    tok = torch.zeros((B, 15), dtype=torch.int32, device=dev)
    emb = torch.zeros((B, g.d_talker), device=dev)
    pred.run(torch.from_numpy(H[0]).to(dev), torch.from_numpy(bad).to(dev), tok, emb)
    torch.cuda.synchronize()
    assert pred.get_error() == 1
    assert pred.get_error() == 0
    np.testing.assert_array_equal(tok.cpu().numpy(), ref["tokens"])
    np.testing.assert_array_equal(emb.cpu().numpy(), ref["embsum"])
    force = np.zeros((B, 15), dtype=np.int32)
    force[2, 6] = -1
    pred.run(torch.from_numpy(H[0]).to(dev), torch.from_numpy(fixed).to(dev), tok, emb,
             force=torch.from_numpy(force).to(dev))
    torch.cuda.synchronize()
    assert pred.get_error() == 2
    assert pred.get_error() == 0


def test_flow_kernel_record_tags_restart(monkeypatch):
    """The kernel's 32-bit record tags restart, after its records are
    cleared, before they would wrap; frames on both sides of the restart
    equal a fresh handle's bit for bit."""
    wl, W, model, pred = workload("b16")
    ppf = 1 + 15 * (5 * wl.geom.n_layers + 1) + 1
    last = 2**32 - 1 - 2 * ppf
    monkeypatch.setenv("QP_TEST_EPOCH0", str(last - 50))
    late = bd.Predictor(W, wl.geom, max_batch=16)
    monkeypatch.delenv("QP_TEST_EPOCH0")
    H, q0 = synth.make_inputs(wl.geom, 7, 3, 8500)
    for f in range(3):
        a = gpu_frame(pred, H[f], q0[f])
        b = gpu_frame(late, H[f], q0[f])
        for key in ("tokens", "logits", "embsum"):
            np.testing.assert_array_equal(a[key], b[key])
    late.close()


# ----------------------------------------------------------------------------
# the batched matrix-core path (bf16 / Q8_0 / Q4_0 weights, any B)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_bf16", "tiny_q8ema", "tiny_q4"])
def test_tiled_tiny_all_frames(name):
    wl, W, model, pred = workload(name)
    H, q0 = synth.make_inputs(wl.geom, wl.batch, wl.frames, wl.input_seed)
    rows = np.arange(wl.batch)
    for f in range(wl.frames):
        check_against_oracle(name, model, pred, H[f], q0[f], rows, tiled=True)


@pytest.mark.parametrize("B", [1, 2, 3, 16, 17, 37])
def test_tiled_batch_sizes(B):
    """Row tiles of 16/32/64 with ragged tails, split-K on and off."""
    wl, W, model, pred = workload("tiny_bf16")
    H, q0 = synth.make_inputs(wl.geom, B, 1, 3100 + B)
    check_against_oracle(f"tiled B={B}", model, pred, H[0], q0[0], np.arange(B), tiled=True)


@pytest.mark.parametrize("name", ["tiny_bf16", "tiny_q8ema", "tiny_q4"])
@pytest.mark.parametrize("B", [65, 100, 160])
def test_tiled_large_batches(name, B):
    """Above 64 rows: tiles of two 16-row fragments with ragged tails for
    q/k/v, gate/up and lm_head, one-fragment tiles for the residual products,
    split-K for the projection; every row against the oracle."""
    wl, W, model, _ = workload(name)
    key = name + "_large"
    if key not in _cache:
        _cache[key] = bd.Predictor(W, wl.geom, max_batch=160)
    pred = _cache[key]
    H, q0 = synth.make_inputs(wl.geom, B, 1, 3200 + B)
    check_against_oracle(f"tiled {name} B={B}", model, pred, H[0], q0[0], np.arange(B), tiled=True)


@pytest.mark.parametrize("name", ["tiny", "tiny_bf16"])
def test_zero_layers(name):
    """Degenerate geometry without decoder layers: step k's logits are the
    lm_head of the normed projected-table row (the oracle's zero-layer pin).
    fp32 weights on the generic path (persistent and stepwise), bf16 on the
    batched path."""
    wl = synth.WORKLOADS[name]
    g = dataclasses.replace(wl.geom, n_layers=0)
    W = synth.make_weights(g, wl.weight_seed)
    model = O.OracleModel(W, g)
    pred = bd.Predictor(W, g, max_batch=8)
    H, q0 = synth.make_inputs(g, 5, 1, 6060)
    rows = np.arange(5)
    if name == "tiny":
        check_against_oracle("tiny L=0", model, pred, H[0], q0[0], rows)
        check_against_oracle("tiny L=0 stepwise", model, pred, H[0], q0[0], rows, stepwise=True)
    else:
        check_against_oracle("tiny_bf16 L=0", model, pred, H[0], q0[0], rows, tiled=True)
    pred.close()


def test_tiled_taps_composition_and_repeat():
    wl, W, model, pred = workload("tiny_q8ema")
    H, q0 = synth.make_inputs(wl.geom, 12, 1, 3333)
    ref = O.run_frames(model, H[0], q0[0], want_taps=True)
    force = ref["tokens"].astype(np.int32)
    got = gpu_frame(pred, H[0], q0[0], force=force, taps=True, tiled=True)
    err = np.abs(got["taps"] - ref["taps"]).max()
    print(f"[tiled taps] max-abs {err:.3g}")
    assert err <= TOL["q8_0"]
    again = gpu_frame(pred, H[0], q0[0], force=force, taps=True, tiled=True)
    for key in ("tokens", "logits", "embsum", "taps"):
        np.testing.assert_array_equal(again[key], got[key])
    # a permutation of the same batch (same tiling) reproduces each row bitwise
    perm = np.random.default_rng(5).permutation(12)
    sub = gpu_frame(pred, H[0][perm], q0[0][perm], force=force[perm], tiled=True)
    for key in ("tokens", "logits", "embsum"):
        np.testing.assert_array_equal(sub[key], got[key][perm])


def test_tiled_against_dataflow_b2():
    wl, W, model, pred = workload("b16")
    H, q0 = synth.make_inputs(wl.geom, 2, 1, 5151)
    ref = O.run_frames(model, H[0], q0[0])
    force = ref["tokens"].astype(np.int32)
    a = gpu_frame(pred, H[0], q0[0], force=force)
    b = gpu_frame(pred, H[0], q0[0], force=force, tiled=True)
    lg = np.abs(a["logits"] - b["logits"]).max()
    print(f"[tiled vs dataflow B=2] logits max-abs {lg:.3g}")
    assert lg <= TOL["bf16"]
    assert np.abs(a["embsum"] - b["embsum"]).max() <= TOL["bf16"]


def test_tiled_graph_replays_match_stream_path():
    """Without test hooks the batched path replays the graph its handle
    prepared for the smallest batch bucket holding B rows (extra rows zero);
    every replay, interleaved with eager work, must equal the direct launch
    sequence for exactly B rows."""
    wl, W, model, pred = workload("tiny_q8ema")
    dev = _dev()
    g = wl.geom
    sizes = [3, 17, 3, 37, 5, 9, 17, 3, 40]
    for i, B in enumerate(sizes):
        H, q0 = synth.make_inputs(g, B, 1, 6100 + i)
        graph = gpu_frame(pred, H[0], q0[0], logits=False, tiled=True)
        # eager work on the same stream between replays
        junk = torch.randn(1 << 16, device=dev)
        (junk * 2.0).sum().item()
        direct = gpu_frame(pred, H[0], q0[0], logits=True, tiled=True)
        np.testing.assert_array_equal(graph["tokens"], direct["tokens"])
        np.testing.assert_array_equal(graph["embsum"], direct["embsum"])
        again = gpu_frame(pred, H[0], q0[0], logits=False, tiled=True)
        np.testing.assert_array_equal(again["tokens"], graph["tokens"])
        np.testing.assert_array_equal(again["embsum"], graph["embsum"])


@pytest.mark.parametrize("name", ["tiny_q8ema", "b16"])
def test_prepared_graphs_interleaved_without_sync(name):
    """Frames of ten batch sizes over every bucket of a max_batch-40 handle,
    enqueued back to back on one stream with no synchronisation in between
    (each into its own output buffers), then each against the same frame
    launched directly (logits hook) bit for bit.  On the 1.7B geometry the
    graphs include the layer-0 table path."""
    wl, W, model, pred = workload(name)
    dev = _dev()
    g = wl.geom
    assert pred.max_batch == 40
    sizes = [3, 17, 1, 37, 5, 9, 40, 2, 16, 33]
    pending = []
    for i, B in enumerate(sizes):
        H, q0 = synth.make_inputs(g, B, 1, 6300 + i)
        Ht = torch.from_numpy(H[0]).to(dev)
        qt = torch.from_numpy(q0[0]).to(dev)
        tok = torch.full((B, 15), -1, dtype=torch.int32, device=dev)
        emb = torch.full((B, g.d_talker), float("nan"), device=dev)
        pred.run(Ht, qt, tok, emb, tiled=True)
        pending.append((H[0], q0[0], tok, emb))
    torch.cuda.synchronize()
    assert pred.get_error() == 0
    for H, q0, tok, emb in pending:
        direct = gpu_frame(pred, H, q0, logits=True, tiled=True)
        np.testing.assert_array_equal(tok.cpu().numpy(), direct["tokens"])
        np.testing.assert_array_equal(emb.cpu().numpy(), direct["embsum"])


@pytest.mark.parametrize("name,tiled", [("tiny_bf16", True), ("b16", True), ("b16", False)],
                         ids=["batched", "batched-table", "dataflow"])
def test_flags_on_fast_paths(name, tiled):
    """Out-of-range q0 (graph and direct launches) and forced tokens raise the
    sticky flag, are read as token 0, and leave the next call clean.  On the
    1.7B geometry the batched path decides tokens in the next step's layer-0
    attention (the layer-0 table), elsewhere in k_next."""
    wl, W, model, pred = workload(name)
    dev = _dev()
    g = wl.geom
    B = 3 if tiled else 2
    H, q0 = synth.make_inputs(g, B, 1, 8800)
    bad = q0[0].copy()
    bad[B - 1] = -5
    fixed = bad.copy()
    fixed[B - 1] = 0
    ref = gpu_frame(pred, H[0], fixed, logits=False, tiled=tiled)
    Ht = torch.from_numpy(H[0]).to(dev)
    tok = torch.zeros((B, 15), dtype=torch.int32, device=dev)
    emb = torch.zeros((B, g.d_talker), device=dev)
    for hooks in (False, True):
        lg = torch.zeros((B, 15, g.vocab), device=dev) if hooks else None
        pred.run(Ht, torch.from_numpy(bad).to(dev), tok, emb, logits_out=lg, tiled=tiled)
        torch.cuda.synchronize()
        assert pred.get_error() == 1
        assert pred.get_error() == 0
        np.testing.assert_array_equal(tok.cpu().numpy(), ref["tokens"])
        np.testing.assert_array_equal(emb.cpu().numpy(), ref["embsum"])
    force = np.zeros((B, 15), dtype=np.int32)
    force[0, 4] = g.vocab
    ft = torch.from_numpy(force).to(dev)
    pred.run(Ht, torch.from_numpy(fixed).to(dev), tok, emb, force=ft, tiled=tiled)
    torch.cuda.synchronize()
    assert pred.get_error() == 2
    assert pred.get_error() == 0


def test_tiled_full_max_batch():
    wl, W, model, pred = workload("tiny_bf16")
    B = pred.max_batch
    H, q0 = synth.make_inputs(wl.geom, B, 1, 9901)
    rows = np.array([0, B // 2, B - 1])
    check_against_oracle("tiled B=max", model, pred, H[0], q0[0], rows, tiled=True)


def test_q4_generic_path_and_full_size():
    """Q4_0 on the generic path (int8 codes) against the oracle, the batched
    path against it within tolerance, and the 1.7B-shaped Q4_0 workload on
    sampled rows."""
    wl, W, model, pred = workload("tiny_q4")
    H, q0 = synth.make_inputs(wl.geom, 4, 1, 7300)
    ref, got = check_against_oracle("tiny_q4 generic", model, pred, H[0], q0[0], np.arange(4))
    tiled = gpu_frame(pred, H[0], q0[0], force=ref["tokens"].astype(np.int32), tiled=True)
    assert np.abs(tiled["logits"] - got["logits"]).max() <= TOL["q4_0"]
    wl, W, model, pred = workload("q4_b16")
    H, q0 = synth.make_inputs(wl.geom, wl.batch, 2, wl.input_seed)
    check_against_oracle("q4_b16", model, pred, H[1], q0[1], np.array([0, 9, 15]))


@pytest.mark.parametrize("name", ["tiny_q8ema", "tiny_q4"])
def test_small_batches_with_block_formats_take_the_batched_path(name):
    """B <= 2 with Q8_0 or Q4_0 weights on a geometry the dataflow kernel does
    not take (it is built for the 1.7B one) runs on the batched matrix-core
    path by default, not on the generic fp32 kernel: the default call equals
    an explicitly batched one bit for bit, and the oracle within tolerance."""
    wl, W, model, pred = workload(name)
    H, q0 = synth.make_inputs(wl.geom, 2, 1, 9100)
    for B in (1, 2):
        d = gpu_frame(pred, H[0][:B], q0[0][:B], logits=False)
        t = gpu_frame(pred, H[0][:B], q0[0][:B], logits=False, tiled=True)
        np.testing.assert_array_equal(d["tokens"], t["tokens"])
        np.testing.assert_array_equal(d["embsum"], t["embsum"])
    check_against_oracle(f"{name} B=1", model, pred, H[0][:1], q0[0][:1], np.arange(1))
