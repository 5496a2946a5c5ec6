"""Repeat-run determinism on the GPU: one fixed input, a thousand frames in a
row, every output bitwise equal to the first.

The drivers exchange values between workgroups through relaxed device-scope
records (the dataflow kernel) and arrival counters (split K on the batched
path); a lost update, a stale read or a tag mix-up would show as a frame that
differs from its neighbours.  Each case prints its name before it starts and
stops at the first differing frame (checked in groups of 100 on the device).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from rvq_codebook_code_amd import binding as bd
from rvq_codebook_code_amd import synth

pytestmark = pytest.mark.gpu

FRAMES = 1000
GROUP = 100


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _soak(pred, g, B, seed, logits, frames=FRAMES):
    dev = _dev()
    H, q0 = synth.make_inputs(g, B, 1, seed)
    Ht = torch.from_numpy(H[0]).to(dev)
    qt = torch.from_numpy(q0[0]).to(dev)

    def outputs():
        tok = torch.full((B, 15), -1, dtype=torch.int32, device=dev)
        emb = torch.full((B, g.d_talker), float("nan"), device=dev)
        lg = torch.full((B, 15, g.vocab), float("nan"), device=dev) if logits else None
        return tok, emb, lg

    t0, e0, l0 = outputs()
    pred.run(Ht, qt, t0, e0, logits_out=l0)
    torch.cuda.synchronize()
    assert pred.get_error() == 0
    t1, e1, l1 = outputs()
    bad = torch.zeros((), dtype=torch.int64, device=dev)
    done = 0
    while done < frames:
        for _ in range(GROUP):
            pred.run(Ht, qt, t1, e1, logits_out=l1)
            ok = (t1 == t0).all() & (e1.view(torch.int32) == e0.view(torch.int32)).all()
            if logits:
                ok = ok & (l1.view(torch.int32) == l0.view(torch.int32)).all()
            bad += (~ok).to(torch.int64)
        done += GROUP
        torch.cuda.synchronize()
        assert pred.get_error() == 0
        n_bad = int(bad.item())
        assert n_bad == 0, f"{n_bad} of the frames up to {done} differ from the first"
    return t0.cpu().numpy()


@pytest.mark.parametrize("B", [1, 2])
def test_dataflow_kernel_thousand_frames_bitwise(B):
    """The small-batch dataflow kernel (1.7B geometry, bf16), tokens, logits
    and embsum of 1,000 frames of one input."""
    wl = synth.WORKLOADS["b1"]
    print(f"[soak] dataflow B={B}: {FRAMES} frames", flush=True)
    W = synth.make_weights(wl.geom, wl.weight_seed)
    pred = bd.Predictor(W, wl.geom, max_batch=B)
    tok = _soak(pred, wl.geom, B, 5300 + B, logits=True)
    assert len(np.unique(tok)) > 5
    pred.close()


def test_moderate_batch_kernel_thousand_frames_bitwise():
    """The moderate-batch dataflow kernel at B = 16 (the bench's b16
    configuration): tokens, logits and embsum of 1,000 frames of one input."""
    wl = synth.WORKLOADS["b16"]
    print(f"[soak] moderate-batch dataflow B=16: {FRAMES} frames", flush=True)
    W = synth.make_weights(wl.geom, wl.weight_seed)
    pred = bd.Predictor(W, wl.geom, max_batch=wl.batch)
    tok = _soak(pred, wl.geom, wl.batch, 5350, logits=True)
    assert len(np.unique(tok)) > 50
    pred.close()


def test_batched_graph_thousand_frames_bitwise():
    """The batched matrix-core path at B = 128 (the bench's configuration):
    1,000 graph replays (no hooks), tokens and embsum bitwise; then 200
    direct launches with the logits hook, logits included."""
    wl = synth.WORKLOADS["b128"]
    print(f"[soak] batched B=128: {FRAMES} graph frames", flush=True)
    W = synth.make_weights(wl.geom, wl.weight_seed)
    pred = bd.Predictor(W, wl.geom, max_batch=wl.batch)
    tok = _soak(pred, wl.geom, wl.batch, 5400, logits=False)
    assert len(np.unique(tok)) > 100
    print("[soak] batched B=128: direct launches with logits", flush=True)
    _soak(pred, wl.geom, wl.batch, 5401, logits=True, frames=200)
    pred.close()
