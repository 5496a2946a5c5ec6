"""The C ABI on the CPU: the library loads, exports every function qp.h
declares, and rejects bad arguments before touching the GPU."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from rvq_codebook_code_amd import binding as bd
from rvq_codebook_code_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions(name="qp.h"):
    text = open(os.path.join(ROOT, "include", name)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qp_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return bd.load_library()


def test_every_declared_function_is_exported(lib):
    names = header_functions()
    assert set(names) >= {"qp_create", "qp_run_frames", "qp_run_frames_ex", "qp_get_error", "qp_destroy"}
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(bd.EXPORTED) == names


def test_status_strings(lib):
    for st in range(-8, 1):
        s = lib.qp_status_string(st)
        assert s and s != b"unknown status"
    assert lib.qp_status_string(-99) == b"unknown status"


def test_null_handle_calls_fail_cleanly(lib):
    lib.qp_destroy(None)
    st = lib.qp_run_frames(None, 1, None, None, None, None, None)
    assert st == bd.QP_ERR_INVALID_ARG
    assert lib.qp_get_error(None) == bd.QP_ERR_INVALID_ARG
    assert lib.qp_last_device_flags(None) == 0
    assert b"NULL" in lib.qp_last_error()


def _tiny():
    return synth.scaled_geometry(synth.WORKLOADS["tiny"].geom)


@pytest.mark.parametrize("field,value,status", [
    ("n_codebooks", 8, bd.QP_ERR_GEOMETRY),
    ("n_kv_heads", 3, bd.QP_ERR_GEOMETRY),
    ("head_dim", 96, bd.QP_ERR_GEOMETRY),
    ("d_model", 0, bd.QP_ERR_GEOMETRY),
    ("max_batch", 0, bd.QP_ERR_GEOMETRY),
    ("rms_eps", 0.0, bd.QP_ERR_GEOMETRY),
    ("weight_dtype", 7, bd.QP_ERR_DTYPE),
    ("emb_format", 9, bd.QP_ERR_DTYPE),
    ("d_ffn", 772, bd.QP_ERR_SHAPE),
])
def test_geometry_validation(lib, field, value, status):
    g = bd.make_geometry(_tiny(), 4)
    setattr(g, field, value)
    w = bd.QpWeights()
    h = C.c_void_p(123)
    assert lib.qp_create(C.byref(w), C.byref(g), 0, C.byref(h)) == status
    assert h.value is None
    assert lib.qp_last_error()


@pytest.mark.parametrize("dtype", ["q8_0", "q4_0"])
def test_block_formats_need_32_aligned_widths(lib, dtype):
    g = bd.make_geometry(synth.scaled_geometry(_tiny(), weight_dtype=dtype, d_ffn=776), 4)
    h = C.c_void_p()
    assert lib.qp_create(C.byref(bd.QpWeights()), C.byref(g), 0, C.byref(h)) == bd.QP_ERR_SHAPE


def test_missing_weights_rejected(lib):
    geom = _tiny()
    W = synth.make_weights(geom, 5)
    hw = bd._HostWeights(W)
    hw.w.lm_head[7] = None
    g = bd.make_geometry(geom, 4)
    h = C.c_void_p()
    assert lib.qp_create(C.byref(hw.w), C.byref(g), 0, C.byref(h)) == bd.QP_ERR_INVALID_ARG
    hw2 = bd._HostWeights(W)
    hw2.w.layers[1].w_up = None
    assert lib.qp_create(C.byref(hw2.w), C.byref(g), 0, C.byref(h)) == bd.QP_ERR_INVALID_ARG


def test_null_out_pointer(lib):
    g = bd.make_geometry(_tiny(), 4)
    assert lib.qp_create(C.byref(bd.QpWeights()), C.byref(g), 0, None) == bd.QP_ERR_INVALID_ARG


def test_sampling_arguments_rejected_before_the_gpu(lib):
    """Bad sampling parameters and shapes fail with INVALID_ARG without a
    device call (rows = 0 and NULL pointers never reach a launch)."""
    sp = bd.QpSampling(1.0, 0, 1.0)
    assert lib.qp_sample_logits(None, 0, 256, 256, C.byref(sp), None, 1, None, None) == bd.QP_OK
    for bad in (bd.QpSampling(0.0, 0, 1.0), bd.QpSampling(float("nan"), 0, 1.0), bd.QpSampling(float("inf"), 0, 1.0),
                bd.QpSampling(1.0, -1, 1.0), bd.QpSampling(1.0, 0, 0.0), bd.QpSampling(1.0, 0, 1.5),
                bd.QpSampling(1.0, 0, float("nan"))):
        assert lib.qp_sample_logits(None, 0, 256, 256, C.byref(bad), None, 1, None, None) == bd.QP_ERR_INVALID_ARG
    assert lib.qp_sample_logits(None, 0, 256, 256, None, None, 1, None, None) == bd.QP_ERR_INVALID_ARG
    assert lib.qp_sample_logits(None, 0, 0, 256, C.byref(sp), None, 1, None, None) == bd.QP_ERR_INVALID_ARG
    assert lib.qp_sample_logits(None, 0, 4097, 8192, C.byref(sp), None, 1, None, None) == bd.QP_ERR_INVALID_ARG
    assert lib.qp_sample_logits(None, 0, 256, 255, C.byref(sp), None, 1, None, None) == bd.QP_ERR_INVALID_ARG
    assert lib.qp_sample_logits(None, 0, 256, 256, C.byref(sp), None, 0, None, None) == bd.QP_ERR_INVALID_ARG
    assert lib.qp_sample_logits(None, 3, 256, 256, C.byref(sp), None, 1, None, None) == bd.QP_ERR_INVALID_ARG
    assert lib.qp_run_frames_sampled(None, 1, None, None, C.byref(sp), None, None, None, None, None, None) == \
        bd.QP_ERR_INVALID_ARG


def test_talker_functions_exported_and_rejected_before_the_gpu(lib):
    names = header_functions("qp_talker.h")
    assert sorted(bd.EXPORTED_TALKER) == names
    for n in names:
        assert hasattr(lib, n), n
    h = C.c_void_p()
    assert lib.qp_talker_create(None, None, 0, C.byref(h)) == bd.QP_ERR_INVALID_ARG
    assert lib.qp_talker_step(None, 1, None, None, None, 1, None, None, None, None) == bd.QP_ERR_INVALID_ARG
    assert lib.qp_talker_load_history(None, 0, 0, None, None, None) == bd.QP_ERR_INVALID_ARG
    assert lib.qp_talker_get_error(None) == bd.QP_ERR_INVALID_ARG
    lib.qp_talker_destroy(None)


@pytest.mark.parametrize("field,value,status", [
    ("n_q_heads", 24, "QP_ERR_GEOMETRY"),      # neither nkv nor 2*nkv
    ("head_dim", 96, "QP_ERR_GEOMETRY"),
    ("d_model", 2000, "QP_ERR_SHAPE"),
    ("vocab", 3000, "QP_ERR_SHAPE"),
    ("weight_dtype", 0, "QP_ERR_DTYPE"),        # f32 talker weights are not supported
    ("max_ctx", 0, "QP_ERR_GEOMETRY"),
    ("n_slots", 0, "QP_ERR_GEOMETRY"),
])
def test_talker_geometry_validation(lib, field, value, status):
    wl = synth.TALKER_WORKLOADS["talker_tiny"]
    g = wl.geom
    geo = bd.QpTalkerGeometry(g.d_model, g.n_layers, g.n_q_heads, g.n_kv_heads, g.head_dim, g.d_ffn, g.vocab,
                              g.rms_eps, g.rope_base, bd.WEIGHT_DTYPES[g.weight_dtype], 4, 4, 64)
    setattr(geo, field, value)
    w = bd.QpTalkerWeights(None, None, None)
    h = C.c_void_p()
    assert lib.qp_talker_create(C.byref(w), C.byref(geo), 0, C.byref(h)) == getattr(bd, status)
    assert not h.value


_LOG_PROBE = r"""
import ctypes as C, sys
sys.path.insert(0, sys.argv[1])
from rvq_codebook_code_amd import binding as bd, synth
lib = bd.load_library()
g = bd.make_geometry(synth.WORKLOADS["tiny"].geom, 4)
g.n_kv_heads = 3
h = C.c_void_p()
print(lib.qp_create(C.byref(bd.QpWeights()), C.byref(g), 0, C.byref(h)))
"""


@pytest.mark.parametrize("log", [False, True])
def test_failures_print_only_with_qp_log(log):
    """Nothing reaches stderr unless QP_LOG is set; then a failure writes its
    message and status name, one line."""
    import subprocess
    import sys
    env = {k: v for k, v in os.environ.items() if k != "QP_LOG"}
    if log:
        env["QP_LOG"] = "1"
    r = subprocess.run([sys.executable, "-c", _LOG_PROBE, ROOT], env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().splitlines()[-1] == str(bd.QP_ERR_GEOMETRY)
    lines = [l for l in r.stderr.splitlines() if l.startswith("qp: ")]
    if log:
        assert len(lines) == 1, r.stderr
        assert "GEOMETRY" in lines[0].upper(), lines[0]
    else:
        assert lines == []
