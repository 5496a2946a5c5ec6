"""qp_run_frames_noalloc: the same frame as qp_run_frames, with the
small-batch driver's scratch in a static device array.

Two calls in a row (B = 2, then a smaller B = 1 on other inputs) through the
C ABI, each against qp_run_frames on the same inputs bit for bit; bf16 and
Q8_0 + EMA handles, and a handle whose own KV cache has another stride
(max_batch 40).  Then the host-side refusals.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from rvq_codebook_code_amd import binding as bd
from rvq_codebook_code_amd import synth

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _frame(fn, g, H, q0):
    dev = _dev()
    B = H.shape[0]
    tok = torch.full((B, 15), -1, dtype=torch.int32, device=dev)
    emb = torch.full((B, g.d_talker), float("nan"), device=dev)
    fn(torch.from_numpy(np.ascontiguousarray(H)).to(dev), torch.from_numpy(np.ascontiguousarray(q0)).to(dev),
       tok, emb)
    return tok, emb


@pytest.mark.parametrize("name,max_batch", [("b1", 2), ("q8ema", 2), ("b1", 40)])
def test_noalloc_equals_run_frames_on_two_calls(name, max_batch):
    wl = synth.WORKLOADS[name]
    g = wl.geom
    print(f"[noalloc] {name} max_batch={max_batch}", flush=True)
    W = synth.make_weights(g, wl.weight_seed)
    pred = bd.Predictor(W, g, max_batch=max_batch)
    H, q0 = synth.make_inputs(g, 2, 2, 7700 + max_batch)
    for call, B in enumerate((2, 1)):
        # both calls enqueued before either result is read
        t_na, e_na = _frame(pred.run_noalloc, g, H[call][:B], q0[call][:B])
        t_rf, e_rf = _frame(pred.run, g, H[call][:B], q0[call][:B])
        torch.cuda.synchronize()
        assert pred.get_error() == 0
        np.testing.assert_array_equal(t_na.cpu().numpy(), t_rf.cpu().numpy())
        np.testing.assert_array_equal(e_na.cpu().numpy().view(np.int32), e_rf.cpu().numpy().view(np.int32))
        assert (t_na.cpu().numpy() >= 0).all()
    pred.close()


def test_noalloc_refusals_and_flag():
    dev = _dev()
    wl = synth.WORKLOADS["b1"]
    g = wl.geom
    W = synth.make_weights(g, wl.weight_seed)
    pred = bd.Predictor(W, g, max_batch=4)
    H, q0 = synth.make_inputs(g, 3, 1, 7800)
    # B above the static scratch's two requests
    with pytest.raises(bd.QpError) as ei:
        _frame(pred.run_noalloc, g, H[0], q0[0])
    assert ei.value.status == bd.QP_ERR_BATCH
    # an out-of-range q0 raises the handle's sticky flag and is read as 0
    bad = q0[0][:1].copy()
    bad[0] = g.vocab
    t_bad, _ = _frame(pred.run_noalloc, g, H[0][:1], bad)
    torch.cuda.synchronize()
    assert pred.get_error() == 1
    t_zero, _ = _frame(pred.run_noalloc, g, H[0][:1], np.zeros(1, np.int32))
    torch.cuda.synchronize()
    assert pred.get_error() == 0
    np.testing.assert_array_equal(t_bad.cpu().numpy(), t_zero.cpu().numpy())
    pred.close()
    # a handle the dataflow driver cannot run
    tw = synth.WORKLOADS["tiny_bf16"]
    tiny = bd.Predictor(synth.make_weights(tw.geom, tw.weight_seed), tw.geom, max_batch=2)
    Ht, qt = synth.make_inputs(tw.geom, 1, 1, 7801)
    with pytest.raises(bd.QpError) as ei:
        _frame(tiny.run_noalloc, tw.geom, Ht[0], qt[0])
    assert ei.value.status == bd.QP_ERR_INVALID_ARG
    tiny.close()
