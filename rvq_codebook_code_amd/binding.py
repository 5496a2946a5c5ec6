"""Thin ctypes binding over libqp.so (the C ABI in include/qp.h).

Argument marshalling only: every step of the predictor runs in the library's
HIP kernels.  Device buffers are torch tensors on the handle's GPU; the
library only sees their data pointers and the current HIP stream.  There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

from . import synth

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqp.so")

N_CODEBOOKS = 16
N_STEPS = 15

QP_OK = 0
QP_ERR_INVALID_ARG = -1
QP_ERR_GEOMETRY = -2
QP_ERR_SHAPE = -3
QP_ERR_DTYPE = -4
QP_ERR_OOM = -5
QP_ERR_HIP = -6
QP_ERR_BATCH = -7
QP_ERR_DEVICE_FLAG = -8

QP_FLAG_STEPWISE = 0x1
QP_FLAG_GENERIC = 0x2
QP_FLAG_TILED = 0x4
QP_FLAG_FLOW = 0x8

WEIGHT_DTYPES = {"f32": 0, "bf16": 1, "q8_0": 2, "q4_0": 3}
EMB_FORMATS = {"f32": 0, "bf16": 1, "ema": 2}

EXPORTED = ["qp_create", "qp_run_frames", "qp_run_frames_ex", "qp_run_frames_noalloc", "qp_run_frames_sampled",
            "qp_sample_logits", "qp_get_error", "qp_last_device_flags", "qp_destroy", "qp_status_string",
            "qp_last_error"]
# include/qp_talker.h
EXPORTED_TALKER = ["qp_talker_create", "qp_talker_load_history", "qp_talker_step", "qp_talker_get_error",
                   "qp_talker_last_device_flags", "qp_talker_destroy"]


class QpGeometry(C.Structure):
    _fields_ = [("d_talker", C.c_int32), ("d_model", C.c_int32), ("n_layers", C.c_int32),
                ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("d_ffn", C.c_int32), ("vocab", C.c_int32), ("n_codebooks", C.c_int32),
                ("rms_eps", C.c_float), ("rope_base", C.c_float), ("weight_dtype", C.c_int32),
                ("emb_format", C.c_int32), ("max_batch", C.c_int32)]


class QpLayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "wo", "q_norm", "k_norm",
                                          "ffn_norm", "w_gate", "w_up", "w_down")]


class QpWeights(C.Structure):
    _fields_ = [("proj_w", C.c_void_p), ("proj_b", C.c_void_p),
                ("emb", C.c_void_p * N_CODEBOOKS), ("ema_sum", C.c_void_p * N_CODEBOOKS),
                ("ema_usage", C.c_void_p * N_CODEBOOKS), ("layers", C.POINTER(QpLayerWeights)),
                ("out_norm", C.c_void_p), ("lm_head", C.c_void_p * N_STEPS)]


class QpSampling(C.Structure):
    _fields_ = [("temperature", C.c_float), ("top_k", C.c_int32), ("top_p", C.c_float)]


class QpTalkerGeometry(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("n_layers", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("d_ffn", C.c_int32), ("vocab", C.c_int32),
                ("rms_eps", C.c_float), ("rope_base", C.c_float), ("weight_dtype", C.c_int32),
                ("max_batch", C.c_int32), ("n_slots", C.c_int32), ("max_ctx", C.c_int32)]


class QpTalkerWeights(C.Structure):
    _fields_ = [("layers", C.c_void_p), ("output_norm", C.c_void_p), ("codec_head", C.c_void_p)]


class QpError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__(f"{what}: status {status} ({detail})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> C.CDLL:
    """Load libqp.so (built by ``rvq_codebook_code_amd.build``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m rvq_codebook_code_amd.build`")
    # torch brings its own HIP runtime with the same soname as the system one;
    # load it first so that the library binds to the runtime torch uses
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover
        pass
    lib = C.CDLL(path)
    vp, i32, u32 = C.c_void_p, C.c_int32, C.c_uint32
    lib.qp_create.argtypes = [C.POINTER(QpWeights), C.POINTER(QpGeometry), i32, C.POINTER(vp)]
    lib.qp_create.restype = i32
    lib.qp_run_frames.argtypes = [vp, i32, vp, vp, vp, vp, vp]
    lib.qp_run_frames.restype = i32
    lib.qp_run_frames_ex.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, u32]
    lib.qp_run_frames_ex.restype = i32
    lib.qp_run_frames_noalloc.argtypes = [vp, i32, vp, vp, vp, vp, vp]
    lib.qp_run_frames_noalloc.restype = i32
    lib.qp_run_frames_sampled.argtypes = [vp, i32, vp, vp, C.POINTER(QpSampling), vp, vp, vp, vp, vp, vp]
    lib.qp_run_frames_sampled.restype = i32
    lib.qp_sample_logits.argtypes = [vp, i32, i32, C.c_int64, C.POINTER(QpSampling), vp, i32, vp, vp]
    lib.qp_sample_logits.restype = i32
    lib.qp_talker_create.argtypes = [C.POINTER(QpTalkerWeights), C.POINTER(QpTalkerGeometry), i32, C.POINTER(vp)]
    lib.qp_talker_create.restype = i32
    lib.qp_talker_load_history.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.qp_talker_load_history.restype = i32
    lib.qp_talker_step.argtypes = [vp, i32, vp, vp, vp, i32, vp, vp, vp, vp]
    lib.qp_talker_step.restype = i32
    lib.qp_talker_get_error.argtypes = [vp]
    lib.qp_talker_get_error.restype = i32
    lib.qp_talker_last_device_flags.argtypes = [vp]
    lib.qp_talker_last_device_flags.restype = u32
    lib.qp_talker_destroy.argtypes = [vp]
    lib.qp_talker_destroy.restype = None
    lib.qp_get_error.argtypes = [vp]
    lib.qp_get_error.restype = i32
    lib.qp_last_device_flags.argtypes = [vp]
    lib.qp_last_device_flags.restype = u32
    lib.qp_destroy.argtypes = [vp]
    lib.qp_destroy.restype = None
    lib.qp_status_string.argtypes = [i32]
    lib.qp_status_string.restype = C.c_char_p
    lib.qp_last_error.argtypes = []
    lib.qp_last_error.restype = C.c_char_p
    _lib = lib
    return lib


def _check(lib, st: int, what: str):
    if st != QP_OK:
        raise QpError(st, what, (lib.qp_last_error() or b"").decode())


def make_geometry(geom: synth.Geometry, max_batch: int) -> QpGeometry:
    return QpGeometry(geom.d_talker, geom.d_model, geom.n_layers, geom.n_q_heads, geom.n_kv_heads,
                      geom.head_dim, geom.d_ffn, geom.vocab, geom.n_codebooks, geom.rms_eps,
                      geom.rope_base, WEIGHT_DTYPES[geom.weight_dtype], EMB_FORMATS[geom.emb_format],
                      max_batch)


class _HostWeights:
    """ctypes views of a weight dict; keeps the numpy buffers alive."""

    def __init__(self, W: dict):
        self._keep = []

        def ptr(a):
            if a is None:
                return None
            a = np.ascontiguousarray(a)
            self._keep.append(a)
            return a.ctypes.data

        w = QpWeights()
        w.proj_w = ptr(W["proj_w"])
        w.proj_b = ptr(W["proj_b"])
        if W["emb_format"] == "ema":
            for j in range(N_CODEBOOKS):
                w.ema_sum[j] = ptr(W["ema_sum"][j])
                w.ema_usage[j] = ptr(W["ema_usage"][j])
        else:
            for j in range(N_CODEBOOKS):
                w.emb[j] = ptr(W["emb"][j])
        n = len(W["layers"])
        arr = (QpLayerWeights * max(n, 1))()
        for i, lw in enumerate(W["layers"]):
            for f, _ in QpLayerWeights._fields_:
                setattr(arr[i], f, ptr(lw[f]))
        self._keep.append(arr)
        w.layers = C.cast(arr, C.POINTER(QpLayerWeights))
        w.out_norm = ptr(W["out_norm"])
        for k in range(N_STEPS):
            w.lm_head[k] = ptr(W["lm_head"][k])
        self.w = w


def _dptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


class Predictor:
    """One ``qp_handle``: weights resident on one GPU, scratch for max_batch."""

    def __init__(self, W: dict, geom: synth.Geometry, max_batch: int, device: int = 0):
        self.lib = load_library()
        self.geom = geom
        self.max_batch = max_batch
        self.device = device
        hw = _HostWeights(W)
        g = make_geometry(geom, max_batch)
        h = C.c_void_p()
        _check(self.lib, self.lib.qp_create(C.byref(hw.w), C.byref(g), device, C.byref(h)), "qp_create")
        self.h = h

    def run(self, H, q0, tokens_out, embsum_out, force=None, logits_out=None, taps_out=None,
            stepwise: bool = False, generic: bool = False, tiled: bool = False, flow: bool = False, stream=None):
        """Enqueue one frame on ``stream`` (default: torch's current stream)."""
        import torch
        B = H.shape[0]
        for t in (H, q0, tokens_out, embsum_out, force, logits_out, taps_out):
            if t is not None:
                assert t.is_cuda and t.is_contiguous()
        assert H.dtype == torch.float32 and q0.dtype == torch.int32
        assert tokens_out.dtype == torch.int32 and embsum_out.dtype == torch.float32
        assert tuple(H.shape) == (B, self.geom.d_talker) and tuple(q0.shape) == (B,)
        assert tuple(tokens_out.shape) == (B, N_STEPS) and tuple(embsum_out.shape) == (B, self.geom.d_talker)
        if force is not None:
            assert force.dtype == torch.int32 and tuple(force.shape) == (B, N_STEPS)
        if logits_out is not None:
            assert logits_out.dtype == torch.float32 and tuple(logits_out.shape) == (B, N_STEPS, self.geom.vocab)
        if taps_out is not None:
            assert taps_out.dtype == torch.float32
            assert tuple(taps_out.shape) == (N_CODEBOOKS, self.geom.n_layers, B, self.geom.d_model)
        if stream is None:
            stream = torch.cuda.current_stream(H.device).cuda_stream
        flags = ((QP_FLAG_STEPWISE if stepwise else 0) | (QP_FLAG_GENERIC if generic else 0) |
                 (QP_FLAG_TILED if tiled else 0) | (QP_FLAG_FLOW if flow else 0))
        if force is None and logits_out is None and taps_out is None and flags == 0:
            st = self.lib.qp_run_frames(self.h, B, _dptr(H), _dptr(q0), _dptr(tokens_out),
                                        _dptr(embsum_out), stream)
        else:
            st = self.lib.qp_run_frames_ex(self.h, B, _dptr(H), _dptr(q0), _dptr(tokens_out),
                                           _dptr(embsum_out), stream, _dptr(force), _dptr(logits_out),
                                           _dptr(taps_out), flags)
        _check(self.lib, st, "qp_run_frames")

    def run_noalloc(self, H, q0, tokens_out, embsum_out, stream=None):
        """Enqueue one frame through qp_run_frames_noalloc (static device
        scratch; B <= 2 on the dataflow driver)."""
        import torch
        B = H.shape[0]
        for t in (H, q0, tokens_out, embsum_out):
            assert t.is_cuda and t.is_contiguous()
        assert H.dtype == torch.float32 and q0.dtype == torch.int32
        assert tokens_out.dtype == torch.int32 and embsum_out.dtype == torch.float32
        assert tuple(H.shape) == (B, self.geom.d_talker) and tuple(q0.shape) == (B,)
        assert tuple(tokens_out.shape) == (B, N_STEPS) and tuple(embsum_out.shape) == (B, self.geom.d_talker)
        if stream is None:
            stream = torch.cuda.current_stream(H.device).cuda_stream
        st = self.lib.qp_run_frames_noalloc(self.h, B, _dptr(H), _dptr(q0), _dptr(tokens_out), _dptr(embsum_out),
                                            stream)
        _check(self.lib, st, "qp_run_frames_noalloc")

    def run_sampled(self, H, q0, uniforms, tokens_out, embsum_out, temperature: float, top_k: int = 0,
                    top_p: float = 1.0, force=None, logits_out=None, stream=None):
        """Enqueue one frame whose tokens are drawn (temperature, top-k,
        top-p) with the caller's uniforms [B, 15] instead of the argmax."""
        import torch
        B = H.shape[0]
        for t in (H, q0, uniforms, tokens_out, embsum_out, force, logits_out):
            if t is not None:
                assert t.is_cuda and t.is_contiguous()
        assert H.dtype == torch.float32 and q0.dtype == torch.int32 and uniforms.dtype == torch.float32
        assert tuple(uniforms.shape) == (B, N_STEPS)
        assert tuple(H.shape) == (B, self.geom.d_talker) and tuple(q0.shape) == (B,)
        assert tuple(tokens_out.shape) == (B, N_STEPS) and tuple(embsum_out.shape) == (B, self.geom.d_talker)
        if force is not None:
            assert force.dtype == torch.int32 and tuple(force.shape) == (B, N_STEPS)
        if logits_out is not None:
            assert logits_out.dtype == torch.float32 and tuple(logits_out.shape) == (B, N_STEPS, self.geom.vocab)
        if stream is None:
            stream = torch.cuda.current_stream(H.device).cuda_stream
        sp = QpSampling(temperature, top_k, top_p)
        st = self.lib.qp_run_frames_sampled(self.h, B, _dptr(H), _dptr(q0), C.byref(sp), _dptr(uniforms),
                                            _dptr(tokens_out), _dptr(embsum_out), stream, _dptr(force),
                                            _dptr(logits_out))
        _check(self.lib, st, "qp_run_frames_sampled")

    def get_error(self) -> int:
        """Synchronise; returns 0 or the raw device flag bits (and clears them)."""
        st = self.lib.qp_get_error(self.h)
        if st == QP_OK:
            return 0
        if st == QP_ERR_DEVICE_FLAG:
            return int(self.lib.qp_last_device_flags(self.h))
        _check(self.lib, st, "qp_get_error")
        return 0

    def close(self):
        if getattr(self, "h", None):
            self.lib.qp_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def sample_logits(logits, uniforms, tokens_out, temperature: float, top_k: int = 0, top_p: float = 1.0,
                  stream=None):
    """Draw one token per row of logits [rows, V] (device fp32) with
    uniforms [rows] into tokens_out [rows] (int32), on the GPU."""
    import torch
    lib = load_library()
    rows, V = logits.shape
    for t in (logits, uniforms, tokens_out):
        assert t.is_cuda
    assert logits.dtype == torch.float32 and logits.stride(1) == 1
    assert uniforms.dtype == torch.float32 and tuple(uniforms.shape) == (rows,) and uniforms.is_contiguous()
    assert tokens_out.dtype == torch.int32 and tuple(tokens_out.shape) == (rows,) and tokens_out.is_contiguous()
    if stream is None:
        stream = torch.cuda.current_stream(logits.device).cuda_stream
    sp = QpSampling(temperature, top_k, top_p)
    st = lib.qp_sample_logits(_dptr(logits), rows, V, logits.stride(0), C.byref(sp), _dptr(uniforms), 1,
                              _dptr(tokens_out), stream)
    _check(lib, st, "qp_sample_logits")


class Talker:
    """One ``qp_talker``: Talker weights resident on one GPU, a bf16 KV cache
    of n_slots x max_ctx positions, scratch for max_batch rows."""

    def __init__(self, W: dict, geom, max_batch: int, n_slots: int, max_ctx: int, device: int = 0):
        self.lib = load_library()
        self.geom = geom
        self.max_batch, self.n_slots, self.max_ctx = max_batch, n_slots, max_ctx
        keep = []

        def ptr(a):
            a = np.ascontiguousarray(a)
            keep.append(a)
            return a.ctypes.data

        n = len(W["layers"])
        arr = (QpLayerWeights * max(n, 1))()
        for i, lw in enumerate(W["layers"]):
            for f, _ in QpLayerWeights._fields_:
                setattr(arr[i], f, ptr(lw[f]))
        w = QpTalkerWeights(C.cast(arr, C.c_void_p), ptr(W["output_norm"]), ptr(W["codec_head"]))
        g = QpTalkerGeometry(geom.d_model, geom.n_layers, geom.n_q_heads, geom.n_kv_heads, geom.head_dim,
                             geom.d_ffn, geom.vocab, geom.rms_eps, geom.rope_base, WEIGHT_DTYPES[geom.weight_dtype],
                             max_batch, n_slots, max_ctx)
        h = C.c_void_p()
        _check(self.lib, self.lib.qp_talker_create(C.byref(w), C.byref(g), device, C.byref(h)), "qp_talker_create")
        self.h = h

    def load_history(self, slot: int, K, V, stream=None):
        """K, V: device uint16 (bf16 bits) [L, n, nkv, hd] of positions 0..n-1."""
        import torch
        n = 0 if K is None else K.shape[1]
        if K is not None:
            assert K.is_cuda and K.is_contiguous() and V.is_contiguous() and K.dtype == torch.int16
            assert tuple(K.shape) == tuple(V.shape)
        if stream is None:
            stream = torch.cuda.current_stream().cuda_stream
        _check(self.lib, self.lib.qp_talker_load_history(self.h, slot, n, _dptr(K), _dptr(V), stream),
               "qp_talker_load_history")

    def step(self, x, slots, pos, max_len: int, H_out, q0_out, logits_out=None, stream=None):
        """Enqueue one decode step for B = x.shape[0] requests."""
        import torch
        B = x.shape[0]
        for t in (x, slots, pos, H_out, q0_out, logits_out):
            if t is not None:
                assert t.is_cuda and t.is_contiguous()
        assert x.dtype == torch.float32 and tuple(x.shape) == (B, self.geom.d_model)
        assert slots.dtype == torch.int32 and pos.dtype == torch.int32 and tuple(slots.shape) == (B,)
        assert H_out.dtype == torch.float32 and tuple(H_out.shape) == (B, self.geom.d_model)
        assert q0_out.dtype == torch.int32 and tuple(q0_out.shape) == (B,)
        if logits_out is not None:
            assert logits_out.dtype == torch.float32 and tuple(logits_out.shape) == (B, self.geom.vocab)
        if stream is None:
            stream = torch.cuda.current_stream(x.device).cuda_stream
        st = self.lib.qp_talker_step(self.h, B, _dptr(x), _dptr(slots), _dptr(pos), max_len, _dptr(H_out),
                                     _dptr(q0_out), _dptr(logits_out), stream)
        _check(self.lib, st, "qp_talker_step")

    def get_error(self) -> int:
        st = self.lib.qp_talker_get_error(self.h)
        if st == QP_OK:
            return 0
        if st == QP_ERR_DEVICE_FLAG:
            return int(self.lib.qp_talker_last_device_flags(self.h))
        _check(self.lib, st, "qp_talker_get_error")
        return 0

    def close(self):
        if getattr(self, "h", None):
            self.lib.qp_talker_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
