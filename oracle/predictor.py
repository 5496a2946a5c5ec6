"""CPU oracle for the Qwen3-TTS Code Predictor ("Subcode") loop.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the GPU library and never calls it.

Plain, slow and written to be checked by eye: float64 NumPy throughout, one
position at a time, one layer at a time, one head at a time.  Matrix products
use NumPy's ``@`` as the only library primitive.

What it computes, per request and per audio frame (sources: the pages'
descriptions of the model and of the exported predictor):

* The Talker emits a frame hidden state H and the first codebook token q0;
  the Code Predictor then emits the remaining 15 codebook tokens in a fixed
  15-step loop (hackernews.jp translation of the Nari Labs post, section
  "Qwen3-TTSの最適化方法" and its subsection 3; agentlenshq summary,
  "Qwen3-TTS 的架构优化").
* The predictor is stateless across frames, greedy, batched, KV-cached and
  fed by H (mixtureofinsights OpenVINO port, section 2.2).
* Inputs of width dT (H and every codebook embedding row) go through
  ``small_to_mtp_projection`` (weight and bias) into the predictor width dP;
  the codebook tables ``codec_embd.{0..14}`` are in the Talker width and the
  heads ``lm_head.{0..14}`` in the predictor width (rightkit-qts exporter
  README, "Loader contract" table and "Expected verification shapes").
* Each block has attn_norm, attn_q/k/v, attn_output, attn_q_norm,
  attn_k_norm, ffn_norm, ffn_gate, ffn_up, ffn_down, and no other tensors;
  the tensor counts (88 = 36 Q8_0 + 30 F16 + 22 F32) leave room for exactly
  one bias, the projection's (same README, output table and storage policy).
* Frame output: tokens q1..q15 and the sum of the 16 codebook embeddings
  E_0[q0] + ... + E_15[q15] (16 RVQ codebooks: forpes.ru RustTTS article,
  "Компоненты"; the RVQ residual sum: mixtureofinsights section 1).
* EMA codebooks are embedding_sum / (cluster_usage + 1e-7) (forpes.ru,
  "Проблема 1: Формат codebook'ов").
* Q8_0 rows are blocks of 32 along the input dimension, an f16 scale then 32
  int8 codes, value = code * scale (the README's Q8_0 export through gguf).
* Q4_0 (the RustTTS article loads q4_0 GGUF files, "Поддержка
  GGUF-квантизации"; the block layout is read as GGUF's): blocks of 32 along
  the input dimension, an f16 scale then 16 bytes of 4-bit codes (element j
  in the low nibble of byte j, element j + 16 in the high nibble), value =
  (code - 8) * scale.

Readings taken where the pages are silent (each listed with its reason in the
design notes): prefill is [H, E_0[q0]] at positions 0 and 1; positions restart
at 0 every frame; plain rotate-half RoPE; per-head q/k RMSNorm after the
projection and before RoPE with the layer eps; consecutive query heads share a
kv head; argmax takes the lowest index on exact ties and is taken on the
logits rounded to fp32 (the precision the GPU decides in).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np

# ----------------------------------------------------------------------------
# weight materialisation (storage format -> float64)
# ----------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the top half of an IEEE fp32 word."""
    u32 = bits.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def dequant_q8_0(packed: np.ndarray, in_features: int) -> np.ndarray:
    """GGUF Q8_0: each 34-byte block is a little-endian f16 scale d followed
    by 32 signed 8-bit codes q; the 32 values are q * d.  Blocks run along
    the input dimension of a row-major [out, in] matrix."""
    out_f = packed.shape[0]
    nb = in_features // 32
    blocks = packed.reshape(out_f, nb, 34)
    d = blocks[..., 0:2].copy().view(np.float16).astype(np.float64)  # [out, nb, 1]
    q = blocks[..., 2:].copy().view(np.int8).astype(np.float64)      # [out, nb, 32]
    return (q * d).reshape(out_f, in_features)


def dequant_q4_0(packed: np.ndarray, in_features: int) -> np.ndarray:
    """GGUF Q4_0: each 18-byte block is a little-endian f16 scale d followed
    by 16 bytes; byte j carries the 4-bit code of element j (low nibble) and
    of element j + 16 (high nibble), and a code c stands for (c - 8) * d.
    Blocks run along the input dimension of a row-major [out, in] matrix."""
    out_f = packed.shape[0]
    nb = in_features // 32
    blocks = packed.reshape(out_f, nb, 18)
    d = blocks[..., 0:2].copy().view(np.float16).astype(np.float64)  # [out, nb, 1]
    qs = blocks[..., 2:].astype(np.int64)                             # [out, nb, 16]
    codes = np.concatenate([qs & 15, qs >> 4], axis=-1)               # elements 0..15, 16..31
    return ((codes - 8).astype(np.float64) * d).reshape(out_f, in_features)


def materialise_matrix(m: np.ndarray, dtype: str, in_features: int) -> np.ndarray:
    if dtype == "f32":
        return m.astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(m)
    if dtype == "q8_0":
        return dequant_q8_0(m, in_features)
    if dtype == "q4_0":
        return dequant_q4_0(m, in_features)
    raise ValueError(dtype)


def ema_codebook(embedding_sum: np.ndarray, cluster_usage: np.ndarray) -> np.ndarray:
    """EMA codebook table: row v is embedding_sum[v] / (cluster_usage[v] + 1e-7)
    (forpes.ru, "Проблема 1")."""
    s = embedding_sum.astype(np.float64)
    u = cluster_usage.astype(np.float64)
    return s / (u[:, None] + 1e-7)


class OracleModel:
    """Float64 copy of one predictor weight set."""

    def __init__(self, W: dict, geom):
        self.g = geom
        wd = W["weight_dtype"]
        g = geom
        self.proj_w = materialise_matrix(W["proj_w"], wd, g.d_talker)
        self.proj_b = W["proj_b"].astype(np.float64)
        if W["emb_format"] == "ema":
            self.emb = [ema_codebook(s, u) for s, u in zip(W["ema_sum"], W["ema_usage"])]
        elif W["emb_format"] == "bf16":
            self.emb = [bf16_bits_to_f64(e) for e in W["emb"]]
        else:
            self.emb = [e.astype(np.float64) for e in W["emb"]]
        self.layers = []
        for lw in W["layers"]:
            self.layers.append({
                "attn_norm": lw["attn_norm"].astype(np.float64),
                "wq": materialise_matrix(lw["wq"], wd, g.d_model),
                "wk": materialise_matrix(lw["wk"], wd, g.d_model),
                "wv": materialise_matrix(lw["wv"], wd, g.d_model),
                "wo": materialise_matrix(lw["wo"], wd, g.n_q_heads * g.head_dim),
                "q_norm": lw["q_norm"].astype(np.float64),
                "k_norm": lw["k_norm"].astype(np.float64),
                "ffn_norm": lw["ffn_norm"].astype(np.float64),
                "w_gate": materialise_matrix(lw["w_gate"], wd, g.d_model),
                "w_up": materialise_matrix(lw["w_up"], wd, g.d_model),
                "w_down": materialise_matrix(lw["w_down"], wd, g.d_ffn),
            })
        self.out_norm = W["out_norm"].astype(np.float64)
        self.lm_head = [materialise_matrix(m, wd, g.d_model) for m in W["lm_head"]]


# ----------------------------------------------------------------------------
# building blocks
# ----------------------------------------------------------------------------


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """gain * x / sqrt(mean(x^2) + eps) over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return gain * (x / np.sqrt(ms + eps))


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def rope(x: np.ndarray, pos: int, base: float) -> np.ndarray:
    """Rotate-half RoPE on the last axis (length hd): element i pairs with
    i + hd/2 and both turn by the angle pos * base**(-2i/hd)."""
    hd = x.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(pos) * np.power(float(base), -2.0 * i / hd)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def kv_head_of(h: int, n_q: int, n_kv: int) -> int:
    """Consecutive query heads share a kv head."""
    return (h * n_kv) // n_q


def argmax_lowest(logits: np.ndarray) -> np.ndarray:
    """Greedy choice over the last axis, decided on fp32-rounded logits;
    np.argmax returns the first (lowest) index among equal maxima."""
    return np.argmax(logits.astype(np.float32), axis=-1)


def top2_margin(logits: np.ndarray) -> np.ndarray:
    srt = np.sort(logits, axis=-1)
    return srt[..., -1] - srt[..., -2]


# ----------------------------------------------------------------------------
# one position through the layer stack, against a KV cache
# ----------------------------------------------------------------------------


def decode_position(model: OracleModel, x: np.ndarray, pos: int,
                    kcache: np.ndarray, vcache: np.ndarray,
                    taps: Optional[list] = None) -> np.ndarray:
    """Run one position for every request.

    x: [B, dP] input rows at position ``pos``.  kcache/vcache:
    [L, B, P, nkv, hd], slot ``pos`` is written here, slots < pos hold the
    earlier positions of the same frame.  Returns the last layer's output
    [B, dP].  ``taps`` (optional list) receives each layer's output."""
    g = model.g
    B = x.shape[0]
    hd, nq, nkv = g.head_dim, g.n_q_heads, g.n_kv_heads
    scale = 1.0 / math.sqrt(hd)
    x = x.copy()
    for li, lw in enumerate(model.layers):
        a = rms_norm(x, lw["attn_norm"], g.rms_eps)
        q = (a @ lw["wq"].T).reshape(B, nq, hd)
        k = (a @ lw["wk"].T).reshape(B, nkv, hd)
        v = (a @ lw["wv"].T).reshape(B, nkv, hd)
        q = rms_norm(q, lw["q_norm"], g.rms_eps)
        k = rms_norm(k, lw["k_norm"], g.rms_eps)
        q = rope(q, pos, g.rope_base)
        k = rope(k, pos, g.rope_base)
        kcache[li, :, pos] = k
        vcache[li, :, pos] = v
        o = np.zeros((B, nq, hd))
        for h in range(nq):
            kv = kv_head_of(h, nq, nkv)
            keys = kcache[li, :, : pos + 1, kv, :]          # [B, pos+1, hd]
            vals = vcache[li, :, : pos + 1, kv, :]
            s = np.einsum("bd,btd->bt", q[:, h, :], keys) * scale
            s = s - s.max(axis=-1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=-1, keepdims=True)
            o[:, h, :] = np.einsum("bt,btd->bd", p, vals)
        x = x + o.reshape(B, nq * hd) @ lw["wo"].T
        m = rms_norm(x, lw["ffn_norm"], g.rms_eps)
        x = x + (silu(m @ lw["w_gate"].T) * (m @ lw["w_up"].T)) @ lw["w_down"].T
        if taps is not None:
            taps.append(x.copy())
    return x


def project(model: OracleModel, rows: np.ndarray) -> np.ndarray:
    """small_to_mtp_projection: W_p @ row + b_p, from dT to dP."""
    return rows @ model.proj_w.T + model.proj_b


def run_frames(model: OracleModel, H: np.ndarray, q0: np.ndarray,
               force: Optional[np.ndarray] = None,
               want_taps: bool = False,
               sampling: Optional[tuple] = None,
               uniforms: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """One frame for B independent requests.

    H: [B, dT]; q0: [B] in [0, V).  force: None or [B, 15] — under teacher
    forcing the token fed back at step k (k = 1..15) and summed into the
    embedding total is force[:, k-1]; tokens and logits remain the model's own.
    sampling: None (greedy) or (temperature, top_k, top_p) with uniforms
    [B, 15]; step k then draws its token with ``sampling.sample_token`` and
    the uniform uniforms[:, k-1] in place of the argmax.

    Returns dict: tokens [B,15] int64, logits [B,15,V] float64,
    margin [B,15] (top-2 logit gap), embsum [B,dT] float64, with sampling
    also sample_margin [B,15] (the draw's relative margin), and with
    ``want_taps`` the per-(position, layer) outputs [16, L, B, dP].
    """
    from oracle import sampling as S
    g = model.g
    H = np.asarray(H, dtype=np.float64)
    q0 = np.asarray(q0, dtype=np.int64)
    B = H.shape[0]
    assert q0.shape == (B,)
    assert np.all((q0 >= 0) & (q0 < g.vocab))
    n_pos = g.n_codebooks           # positions 0..15 (H, then E_0..E_14 inputs)
    n_steps = g.n_codebooks - 1
    kcache = np.zeros((g.n_layers, B, n_pos, g.n_kv_heads, g.head_dim))
    vcache = np.zeros_like(kcache)
    tokens = np.zeros((B, n_steps), dtype=np.int64)
    logits = np.zeros((B, n_steps, g.vocab))
    smargin = np.full((B, n_steps), np.inf)
    if sampling is not None:
        uniforms = np.asarray(uniforms, dtype=np.float32)
        assert uniforms.shape == (B, n_steps)
    taps = [] if want_taps else None

    # position 0: the projected frame hidden state
    decode_position(model, project(model, H), 0, kcache, vcache, taps)
    # position 1 carries codebook 0
    e = model.emb[0][q0]
    embsum = e.copy()
    prev = q0
    for k in range(1, n_steps + 1):          # step k predicts q_k at position k
        if k > 1:
            e = model.emb[k - 1][prev]
            embsum = embsum + e
        h = decode_position(model, project(model, e), k, kcache, vcache, taps)
        lg = rms_norm(h, model.out_norm, g.rms_eps) @ model.lm_head[k - 1].T
        assert np.all(np.isfinite(lg))
        logits[:, k - 1] = lg
        if sampling is None:
            tokens[:, k - 1] = argmax_lowest(lg)
        else:
            T, K, P = sampling
            for b in range(B):
                tokens[b, k - 1], smargin[b, k - 1], _ = S.sample_token(lg[b], T, K, P, uniforms[b, k - 1])
        prev = tokens[:, k - 1] if force is None else np.asarray(force[:, k - 1], dtype=np.int64)
    embsum = embsum + model.emb[n_steps][prev]
    out = {"tokens": tokens, "logits": logits, "margin": top2_margin(logits),
           "embsum": embsum}
    if sampling is not None:
        out["sample_margin"] = smargin
    if want_taps:
        L = g.n_layers
        out["taps"] = np.stack(taps).reshape(n_pos, L, B, g.d_model)
    return out


# ----------------------------------------------------------------------------
# brute-force variant: no cache, whole prefix recomputed with explicit loops
# ----------------------------------------------------------------------------


def _layer_stack_full(model: OracleModel, X: np.ndarray) -> np.ndarray:
    """Run the layer stack over a whole causal sequence X [T, dP] of one
    request, attention written as explicit loops with an explicit mask."""
    g = model.g
    T = X.shape[0]
    hd, nq, nkv = g.head_dim, g.n_q_heads, g.n_kv_heads
    x = X.copy()
    for lw in model.layers:
        a = rms_norm(x, lw["attn_norm"], g.rms_eps)
        q = rms_norm((a @ lw["wq"].T).reshape(T, nq, hd), lw["q_norm"], g.rms_eps)
        k = rms_norm((a @ lw["wk"].T).reshape(T, nkv, hd), lw["k_norm"], g.rms_eps)
        v = (a @ lw["wv"].T).reshape(T, nkv, hd)
        for t in range(T):
            q[t] = rope(q[t], t, g.rope_base)
            k[t] = rope(k[t], t, g.rope_base)
        o = np.zeros((T, nq, hd))
        for h in range(nq):
            kv = kv_head_of(h, nq, nkv)
            for t in range(T):
                scores = np.full(T, -np.inf)
                for u in range(T):
                    if u <= t:                       # causal mask
                        dot = 0.0
                        for d in range(hd):
                            dot += q[t, h, d] * k[u, kv, d]
                        scores[u] = dot / math.sqrt(hd)
                mx = max(scores[: t + 1])
                w = [math.exp(scores[u] - mx) if u <= t else 0.0 for u in range(T)]
                tot = sum(w)
                for u in range(t + 1):
                    o[t, h] += (w[u] / tot) * v[u, kv]
        x = x + o.reshape(T, nq * hd) @ lw["wo"].T
        m = rms_norm(x, lw["ffn_norm"], g.rms_eps)
        x = x + (silu(m @ lw["w_gate"].T) * (m @ lw["w_up"].T)) @ lw["w_down"].T
    return x


def run_frame_uncached(model: OracleModel, H: np.ndarray, q0: int) -> Dict[str, np.ndarray]:
    """One frame for ONE request with no KV cache: at every step the whole
    sequence [H, E_0[q0], E_1[q1], ...] is rebuilt and re-run causally."""
    g = model.g
    H = np.asarray(H, dtype=np.float64)
    seq = [project(model, H[None])[0], project(model, model.emb[0][q0][None])[0]]
    toks: List[int] = []
    lgs = []
    for k in range(1, g.n_codebooks):
        out = _layer_stack_full(model, np.stack(seq))
        lg = model.lm_head[k - 1] @ rms_norm(out[-1], model.out_norm, g.rms_eps)
        lgs.append(lg)
        t = int(argmax_lowest(lg[None])[0])
        toks.append(t)
        if k < g.n_codebooks - 1:
            seq.append(project(model, model.emb[k][t][None])[0])
    embsum = model.emb[0][q0].copy()
    for j, t in enumerate(toks, start=1):
        embsum = embsum + model.emb[j][t]
    return {"tokens": np.array(toks), "logits": np.stack(lgs), "embsum": embsum}
