"""Seeded synthetic weights and inputs for the code-predictor workloads.

This module only *draws* numbers and packs them into the storage formats the
predictor consumes (fp32, bf16 bit patterns, GGUF-style Q8_0 blocks, raw EMA
codebook statistics).  It holds none of the predictor's arithmetic: no
normalisation, projection, attention, dequantisation or EMA division happens
here.  Both the CPU oracle and the GPU library read what it produces.

Shapes follow the GGUF exporter README for Qwen3-TTS 1.7B ("Expected
verification shapes" table and the predictor geometry paragraph): matrices are
HF row-major ``[out, in]``; the 16 codebook tables live in the Talker width,
the 15 heads in the predictor width.

Workloads (sizes, value distributions):

* ``tiny``   : predictor width 256, 2 layers, 4 q / 2 kv heads of 64, SwiGLU
               768, RMSNorm eps 1e-6, RoPE base 1e4, 16 codebooks x 256,
               talker width 512, fp32 weights; B=4 x 8 frames.
* ``b1``     : the 1.7B-shaped predictor (1024 wide, 5 layers, 16/8 heads of
               128, FFN 3072, RoPE base 1e6, 16 x 2048 codebooks, talker
               width 2048), bf16 weights; B=1 x 256 frames.
* ``b16``    : same predictor, B=16 x 128 frames.
* ``b128``   : same predictor, B=128 x 64 frames.
* ``q8ema``  : same predictor with every linear in Q8_0 and EMA codebooks
               (embedding_sum = z*usage, usage ~ Gamma(2,1)); B=64 x 64.

Matrices, embeddings and the projection bias are N(0, 0.02); RMSNorm gains
are 1 + N(0, 0.02) (a gain of ~0.02 would make every norm degenerate).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

N_CODEBOOKS = 16
N_STEPS = N_CODEBOOKS - 1  # tokens emitted per frame by the predictor


@dataclasses.dataclass(frozen=True)
class Geometry:
    d_talker: int       # dT: width of H and of the codebook tables
    d_model: int        # dP: predictor hidden width
    n_layers: int       # L
    n_q_heads: int      # nq
    n_kv_heads: int     # nkv
    head_dim: int       # hd
    d_ffn: int          # F
    vocab: int          # V, per codebook
    rms_eps: float
    rope_base: float
    weight_dtype: str   # 'f32' | 'bf16' | 'q8_0' | 'q4_0'   (every linear)
    emb_format: str     # 'f32' | 'bf16' | 'ema'    (the 16 codebook tables)
    n_codebooks: int = N_CODEBOOKS


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    geom: Geometry
    batch: int
    frames: int
    weight_seed: int
    input_seed: int
    description: str


_PRED_17B = dict(d_talker=2048, d_model=1024, n_layers=5, n_q_heads=16,
                 n_kv_heads=8, head_dim=128, d_ffn=3072, vocab=2048,
                 rms_eps=1e-6, rope_base=1e6)

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        "tiny",
        Geometry(d_talker=512, d_model=256, n_layers=2, n_q_heads=4,
                 n_kv_heads=2, head_dim=64, d_ffn=768, vocab=256,
                 rms_eps=1e-6, rope_base=1e4, weight_dtype="f32",
                 emb_format="f32"),
        batch=4, frames=8, weight_seed=1001, input_seed=2001,
        description="tiny predictor, fp32 weights, B=4 x 8 frames"),
    "b1": Workload(
        "b1", Geometry(**_PRED_17B, weight_dtype="bf16", emb_format="bf16"),
        batch=1, frames=256, weight_seed=1002, input_seed=2002,
        description="1.7B-shaped predictor, bf16 weights, B=1 x 256 frames"),
    "b16": Workload(
        "b16", Geometry(**_PRED_17B, weight_dtype="bf16", emb_format="bf16"),
        batch=16, frames=128, weight_seed=1003, input_seed=2003,
        description="1.7B-shaped predictor, bf16 weights, B=16 x 128 frames"),
    "b128": Workload(
        "b128", Geometry(**_PRED_17B, weight_dtype="bf16", emb_format="bf16"),
        batch=128, frames=64, weight_seed=1004, input_seed=2004,
        description="1.7B-shaped predictor, bf16 weights, B=128 x 64 frames"),
    "q8ema": Workload(
        "q8ema", Geometry(**_PRED_17B, weight_dtype="q8_0", emb_format="ema"),
        batch=64, frames=64, weight_seed=1005, input_seed=2005,
        description="1.7B-shaped predictor, Q8_0 linears + EMA codebooks, "
                    "B=64 x 64 frames"),
    # small parity cases for the bf16 / Q8_0 paths (the tiny geometry with the
    # 1.7B configurations' storage formats)
    "tiny_bf16": Workload(
        "tiny_bf16",
        Geometry(d_talker=512, d_model=256, n_layers=2, n_q_heads=4,
                 n_kv_heads=2, head_dim=64, d_ffn=768, vocab=256,
                 rms_eps=1e-6, rope_base=1e4, weight_dtype="bf16",
                 emb_format="bf16"),
        batch=20, frames=4, weight_seed=1101, input_seed=2101,
        description="tiny predictor, bf16 weights and tables, B=20 x 4 frames"),
    "tiny_q8ema": Workload(
        "tiny_q8ema",
        Geometry(d_talker=512, d_model=256, n_layers=2, n_q_heads=4,
                 n_kv_heads=2, head_dim=64, d_ffn=768, vocab=256,
                 rms_eps=1e-6, rope_base=1e4, weight_dtype="q8_0",
                 emb_format="ema"),
        batch=20, frames=4, weight_seed=1102, input_seed=2102,
        description="tiny predictor, Q8_0 linears + EMA codebooks, B=20 x 4 frames"),
    "tiny_q4": Workload(
        "tiny_q4",
        Geometry(d_talker=512, d_model=256, n_layers=2, n_q_heads=4,
                 n_kv_heads=2, head_dim=64, d_ffn=768, vocab=256,
                 rms_eps=1e-6, rope_base=1e4, weight_dtype="q4_0",
                 emb_format="bf16"),
        batch=20, frames=4, weight_seed=1103, input_seed=2103,
        description="tiny predictor, Q4_0 linears, bf16 tables, B=20 x 4 frames"),
    # Q4_0 weights on the 1.7B-shaped predictor (the first "next" row)
    "q4_b16": Workload(
        "q4_b16", Geometry(**_PRED_17B, weight_dtype="q4_0", emb_format="bf16"),
        batch=16, frames=64, weight_seed=1006, input_seed=2006,
        description="1.7B-shaped predictor, Q4_0 linears, bf16 tables, B=16 x 64 frames"),
    "q4_b1": Workload(
        "q4_b1", Geometry(**_PRED_17B, weight_dtype="q4_0", emb_format="bf16"),
        batch=1, frames=256, weight_seed=1006, input_seed=2007,
        description="1.7B-shaped predictor, Q4_0 linears, bf16 tables, B=1 x 256 frames"),
}


def scaled_geometry(base: Geometry, **over) -> Geometry:
    """A copy of ``base`` with some fields replaced (for small test cases)."""
    return dataclasses.replace(base, **over)


# ----------------------------------------------------------------------------
# storage-format packing (no model arithmetic)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16.  Inputs are finite draws."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


Q8_BLOCK = 32
Q8_BLOCK_BYTES = 34  # little-endian f16 scale followed by 32 int8


def pack_q8_0(x: np.ndarray) -> np.ndarray:
    """Pack a row-major ``[out, in]`` fp32 matrix into GGUF-style Q8_0 rows.

    Every row becomes ``in/32`` blocks of 34 bytes along ``in``: the f16
    scale d = max|x|/127 (rounded to f16), then 32 int8 codes
    round-half-away(x/d) clamped to [-127, 127] (all zero when d == 0).
    Returns uint8 ``[out, in/32*34]``.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    out_f, in_f = x.shape
    assert in_f % Q8_BLOCK == 0, "Q8_0 needs in-features divisible by 32"
    nb = in_f // Q8_BLOCK
    blk = x.reshape(out_f, nb, Q8_BLOCK).astype(np.float64)
    amax = np.abs(blk).max(axis=-1)
    d16 = (amax / 127.0).astype(np.float16)
    d = d16.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(d[..., None] > 0, blk / d[..., None], 0.0)
    q = np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), -127, 127).astype(np.int8)
    packed = np.empty((out_f, nb, Q8_BLOCK_BYTES), dtype=np.uint8)
    packed[..., 0:2] = d16.view(np.uint8).reshape(out_f, nb, 2)
    packed[..., 2:] = q.view(np.uint8)
    return packed.reshape(out_f, nb * Q8_BLOCK_BYTES)


Q4_BLOCK_BYTES = 18


def pack_q4_0(x: np.ndarray) -> np.ndarray:
    """Pack a row-major ``[out, in]`` fp32 matrix into GGUF-style Q4_0 rows.

    Every row becomes ``in/32`` blocks of 18 bytes along ``in``: the f16
    scale d = max|x|/7 (rounded to f16), then 16 bytes whose byte j holds the
    4-bit code of element j in its low nibble and of element j + 16 in its
    high nibble; a code is c = clamp(round-half-away(x/d), -8, 7) + 8, so the
    value is (c - 8) * d (all codes 8 when d == 0).  Returns uint8
    ``[out, in/32*18]``.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    out_f, in_f = x.shape
    assert in_f % Q8_BLOCK == 0, "Q4_0 needs in-features divisible by 32"
    nb = in_f // Q8_BLOCK
    blk = x.reshape(out_f, nb, Q8_BLOCK).astype(np.float64)
    amax = np.abs(blk).max(axis=-1)
    d16 = (amax / 7.0).astype(np.float16)
    d = d16.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(d[..., None] > 0, blk / d[..., None], 0.0)
    c = (np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), -8, 7) + 8).astype(np.uint8)
    packed = np.empty((out_f, nb, Q4_BLOCK_BYTES), dtype=np.uint8)
    packed[..., 0:2] = d16.view(np.uint8).reshape(out_f, nb, 2)
    packed[..., 2:] = c[..., :16] | (c[..., 16:] << 4)
    return packed.reshape(out_f, nb * Q4_BLOCK_BYTES)


def _matrix(rng: np.random.Generator, out_f: int, in_f: int, dtype: str):
    w = (rng.standard_normal((out_f, in_f), dtype=np.float32) * np.float32(0.02))
    if dtype == "f32":
        return w
    if dtype == "bf16":
        return f32_to_bf16_bits(w)
    if dtype == "q8_0":
        return pack_q8_0(w)
    if dtype == "q4_0":
        return pack_q4_0(w)
    raise ValueError(dtype)


def _gain(rng: np.random.Generator, n: int) -> np.ndarray:
    return (np.float32(1.0) + rng.standard_normal(n, dtype=np.float32)
            * np.float32(0.02)).astype(np.float32)


def make_weights(geom: Geometry, seed: int) -> dict:
    """Draw a full predictor weight set for ``geom``.

    Draw order: proj_w, proj_b, the 16 codebook tables (or, for EMA, each
    table's usage then its N(0,1) direction), then per layer attn_norm, wq,
    wk, wv, wo, q_norm, k_norm, ffn_norm, w_gate, w_up, w_down, then
    out_norm, then lm_head 0..14.
    """
    g = geom
    rng = np.random.default_rng(seed)
    wd = g.weight_dtype
    W: dict = {"weight_dtype": wd, "emb_format": g.emb_format}
    W["proj_w"] = _matrix(rng, g.d_model, g.d_talker, wd)
    W["proj_b"] = (rng.standard_normal(g.d_model, dtype=np.float32)
                   * np.float32(0.02)).astype(np.float32)
    if g.emb_format == "ema":
        sums: List[np.ndarray] = []
        usage: List[np.ndarray] = []
        for _ in range(g.n_codebooks):
            u = rng.gamma(2.0, 1.0, size=g.vocab).astype(np.float32)
            z = rng.standard_normal((g.vocab, g.d_talker), dtype=np.float32)
            sums.append((z * u[:, None]).astype(np.float32))
            usage.append(u)
        W["ema_sum"] = sums
        W["ema_usage"] = usage
    else:
        embs = []
        for _ in range(g.n_codebooks):
            e = rng.standard_normal((g.vocab, g.d_talker), dtype=np.float32) * np.float32(0.02)
            embs.append(e if g.emb_format == "f32" else f32_to_bf16_bits(e))
        W["emb"] = embs
    qd = g.n_q_heads * g.head_dim
    kd = g.n_kv_heads * g.head_dim
    layers = []
    for _ in range(g.n_layers):
        lw = {}
        lw["attn_norm"] = _gain(rng, g.d_model)
        lw["wq"] = _matrix(rng, qd, g.d_model, wd)
        lw["wk"] = _matrix(rng, kd, g.d_model, wd)
        lw["wv"] = _matrix(rng, kd, g.d_model, wd)
        lw["wo"] = _matrix(rng, g.d_model, qd, wd)
        lw["q_norm"] = _gain(rng, g.head_dim)
        lw["k_norm"] = _gain(rng, g.head_dim)
        lw["ffn_norm"] = _gain(rng, g.d_model)
        lw["w_gate"] = _matrix(rng, g.d_ffn, g.d_model, wd)
        lw["w_up"] = _matrix(rng, g.d_ffn, g.d_model, wd)
        lw["w_down"] = _matrix(rng, g.d_model, g.d_ffn, wd)
        layers.append(lw)
    W["layers"] = layers
    W["out_norm"] = _gain(rng, g.d_model)
    W["lm_head"] = [_matrix(rng, g.vocab, g.d_model, wd) for _ in range(g.n_codebooks - 1)]
    return W


def make_inputs(geom: Geometry, batch: int, frames: int, seed: int):
    """H ``[frames, batch, dT]`` ~ N(0,1) fp32, then q0 ``[frames, batch]``
    int32 uniform in [0, V)."""
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((frames, batch, geom.d_talker), dtype=np.float32)
    q0 = rng.integers(0, geom.vocab, size=(frames, batch), dtype=np.int64).astype(np.int32)
    return H, q0


def make_uniforms(batch: int, frames: int, seed: int):
    """The caller's draws for sampled frames: ``[frames, batch, 15]`` fp32
    uniform in [0, 1), one per request and step."""
    rng = np.random.default_rng(seed)
    return rng.random((frames, batch, 15), dtype=np.float32)


def workload_data(name: str, frames: Optional[int] = None, batch: Optional[int] = None):
    """(workload, weights, H, q0) for a named workload; ``frames``/``batch``
    may shrink the input draw (the weights are always the full set)."""
    wl = WORKLOADS[name]
    W = make_weights(wl.geom, wl.weight_seed)
    H, q0 = make_inputs(wl.geom, batch or wl.batch, frames or wl.frames, wl.input_seed)
    return wl, W, H, q0


# ----------------------------------------------------------------------------
# the Talker decode step (the step before the predictor)
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class TalkerGeometry:
    d_model: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int            # codec head rows (codebook-0 tokens and specials)
    rms_eps: float
    rope_base: float
    weight_dtype: str     # "bf16" | "q8_0" | "q4_0"


@dataclasses.dataclass(frozen=True)
class TalkerWorkload:
    name: str
    geom: TalkerGeometry
    batch: int
    context: int          # history length of every request before the timed steps
    weight_seed: int
    input_seed: int
    description: str


_TALKER_17B = dict(d_model=2048, n_q_heads=16, n_kv_heads=8, head_dim=128, d_ffn=6144,
                   vocab=3072, rms_eps=1e-6, rope_base=1e6)

TALKER_WORKLOADS: Dict[str, TalkerWorkload] = {
    "talker_tiny": TalkerWorkload(
        "talker_tiny",
        TalkerGeometry(d_model=256, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64, d_ffn=768,
                       vocab=384, rms_eps=1e-6, rope_base=1e4, weight_dtype="bf16"),
        batch=3, context=40, weight_seed=3001, input_seed=4001,
        description="tiny Talker, bf16 weights, B=3, 40 positions of history"),
    "talker_tiny_q8": TalkerWorkload(
        "talker_tiny_q8",
        TalkerGeometry(d_model=256, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64, d_ffn=768,
                       vocab=384, rms_eps=1e-6, rope_base=1e4, weight_dtype="q8_0"),
        batch=3, context=40, weight_seed=3011, input_seed=4011,
        description="tiny Talker, Q8_0 weights, B=3, 40 positions of history"),
    "talker_tiny_q4": TalkerWorkload(
        "talker_tiny_q4",
        TalkerGeometry(d_model=256, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64, d_ffn=768,
                       vocab=384, rms_eps=1e-6, rope_base=1e4, weight_dtype="q4_0"),
        batch=3, context=40, weight_seed=3012, input_seed=4012,
        description="tiny Talker, Q4_0 weights, B=3, 40 positions of history"),
    "talker_wide": TalkerWorkload(
        "talker_wide",
        TalkerGeometry(d_model=2560, n_layers=1, n_q_heads=4, n_kv_heads=2, head_dim=64, d_ffn=768,
                       vocab=384, rms_eps=1e-6, rope_base=1e4, weight_dtype="bf16"),
        batch=3, context=40, weight_seed=3005, input_seed=4005,
        description="one-layer Talker wider than 2048 (the products' RMSNorm row sums and the final "
                    "kernel's row in more than one group of loads), bf16 weights, B=3"),
    "talker_l2": TalkerWorkload(
        "talker_l2", TalkerGeometry(n_layers=2, weight_dtype="bf16", **_TALKER_17B),
        batch=4, context=300, weight_seed=3002, input_seed=4002,
        description="1.7B Talker widths with 2 layers, bf16 weights, B=4, up to 300 positions of history"),
    "talker_b1": TalkerWorkload(
        "talker_b1", TalkerGeometry(n_layers=28, weight_dtype="bf16", **_TALKER_17B),
        batch=1, context=1024, weight_seed=3003, input_seed=4003,
        description="1.7B Talker, bf16 weights, B=1, 1024 positions of history"),
    "talker_b16": TalkerWorkload(
        "talker_b16", TalkerGeometry(n_layers=28, weight_dtype="bf16", **_TALKER_17B),
        batch=16, context=1024, weight_seed=3003, input_seed=4004,
        description="1.7B Talker, bf16 weights, B=16, 1024 positions of history each"),
}


def make_talker_weights(geom: TalkerGeometry, seed: int) -> dict:
    """Draw a Talker weight set.  Layer l draws from its own generator
    (seed, l), in the order attn_norm, wq, wk, wv, wo, q_norm, k_norm,
    ffn_norm, w_gate, w_up, w_down; then output_norm and codec_head from
    (seed, n_layers)."""
    g = geom
    wd = g.weight_dtype
    qd = g.n_q_heads * g.head_dim
    kd = g.n_kv_heads * g.head_dim

    def one_layer(l):
        rng = np.random.default_rng([seed, l])
        lw = {}
        lw["attn_norm"] = _gain(rng, g.d_model)
        lw["wq"] = _matrix(rng, qd, g.d_model, wd)
        lw["wk"] = _matrix(rng, kd, g.d_model, wd)
        lw["wv"] = _matrix(rng, kd, g.d_model, wd)
        lw["wo"] = _matrix(rng, g.d_model, qd, wd)
        lw["q_norm"] = _gain(rng, g.head_dim)
        lw["k_norm"] = _gain(rng, g.head_dim)
        lw["ffn_norm"] = _gain(rng, g.d_model)
        lw["w_gate"] = _matrix(rng, g.d_ffn, g.d_model, wd)
        lw["w_up"] = _matrix(rng, g.d_ffn, g.d_model, wd)
        lw["w_down"] = _matrix(rng, g.d_model, g.d_ffn, wd)
        return lw

    # every layer has its own generator, so the draw is the same however the
    # layers are scheduled
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=8) as ex:
        layers = list(ex.map(one_layer, range(g.n_layers)))
    rng = np.random.default_rng([seed, g.n_layers])
    return {"weight_dtype": wd, "layers": layers, "output_norm": _gain(rng, g.d_model),
            "codec_head": _matrix(rng, g.vocab, g.d_model, wd)}


def make_talker_history(geom: TalkerGeometry, n_pos: int, seed: int):
    """A request's cached history: keys and values of positions 0..n_pos-1 as
    bf16 bit patterns [L, n_pos, nkv, hd] (N(0,1) draws: the scale of keys
    after the per-head norm)."""
    rng = np.random.default_rng(seed)
    shape = (geom.n_layers, n_pos, geom.n_kv_heads, geom.head_dim)
    K = f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    V = f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    return K, V


def make_talker_inputs(geom: TalkerGeometry, batch: int, steps: int, seed: int):
    """Step input rows [steps, batch, d_model] ~ N(0,1) fp32."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((steps, batch, geom.d_model), dtype=np.float32)
