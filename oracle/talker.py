"""CPU oracle for one Talker decode step (the step before the Code Predictor).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the GPU library and never calls it.

What the pages fix:

* The Talker is the long-context autoregressive transformer.  For every audio
  frame it attends over the whole history held in a paged KV cache and yields
  the frame hidden state H and the first codebook token q0; the Code Predictor
  then works only on H (mixtureofinsights OpenVINO port, section 1 diagram and
  sections 2.1-2.2; hackernews.jp translation of the Nari Labs post,
  "Qwen3-TTSの最適化方法").  The history is kept per request in a KV store of
  fixed capacity (forpes.ru RustTTS article, "KV-Cache с блочным хранением").
* 1.7B geometry: width 2048, 28 blocks, 16 query and 8 kv heads of 128, FFN
  6144; the block tensors are the predictor's (attn_norm, attn_q/k/v,
  attn_output, attn_q_norm, attn_k_norm, ffn_norm, ffn_gate/up/down); the
  codec table has 3072 rows of width 2048 (rightkit-qts exporter README,
  "Loader contract", its geometry paragraph and "Expected verification
  shapes"), so the codec head that predicts q0 is taken as 3072 x 2048.

Readings taken where the pages are silent or garbled (each listed with its
reason in the design notes):

* The step's input row (width 2048) is given by the caller: how it is made
  (the previous frame's summed codebook embeddings, text conditioning) is not
  part of this step.
* Positions: the article's multimodal RoPE gives three position streams over
  three sections of the head dimension (its split into thirds cannot be
  literal for a head of 128).  For codec frames the three streams carry the
  same index, and with one frequency ladder over the whole head the sections
  then rotate exactly as plain rotate-half RoPE at the frame's absolute
  position, which is what is computed here.
* H is the final-norm output, the vector the codec head reads; q0 is the
  argmax of the head's logits over all 3072 rows (lowest index on exact ties,
  decided on the fp32-rounded logits).
* The cache holds keys (after the per-head norm and RoPE) and values rounded
  to bf16, the storage a bf16 model keeps; attention reads those rounded
  values.  ``kv_round=False`` keeps them exact (used by one pin).

Plain and slow: float64 NumPy, one request and one head at a time.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np

from oracle.predictor import (argmax_lowest, kv_head_of, materialise_matrix,
                              rms_norm, rope, silu)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 (ties to even) through fp32, as a device
    rounds its fp32 value when it stores bf16."""
    f = np.asarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    r = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


class TalkerOracle:
    """Float64 view of one Talker weight set; layers are materialised on
    demand (and kept when ``keep`` is set), so a 28-layer model can be run one
    layer at a time."""

    def __init__(self, W: dict, geom, keep: bool = True):
        self.g = geom
        self.W = W
        self.keep = keep
        self._layers: Dict[int, dict] = {}
        wd = W["weight_dtype"]
        self.output_norm = W["output_norm"].astype(np.float64)
        self.head = materialise_matrix(W["codec_head"], wd, geom.d_model)

    def layer(self, l: int) -> dict:
        if l in self._layers:
            return self._layers[l]
        g, wd, lw = self.g, self.W["weight_dtype"], self.W["layers"][l]
        out = {
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
        }
        if self.keep:
            self._layers[l] = out
        return out


def decode_step(model: TalkerOracle, x: np.ndarray, pos: int,
                K: np.ndarray, V: np.ndarray, kv_round: bool = True) -> Dict[str, np.ndarray]:
    """One decode step of ONE request.

    x: [d] input row at position ``pos``; K, V: [L, >= pos, nkv, hd] the
    cached keys and values of positions 0 .. pos-1 (bf16-rounded values).
    Returns H [d], logits [vocab], q0, margin (top-2 logit gap) and the new
    cache rows k_new, v_new [L, nkv, hd] for position ``pos``."""
    g = model.g
    hd, nq, nkv = g.head_dim, g.n_q_heads, g.n_kv_heads
    scale = 1.0 / math.sqrt(hd)
    x = np.asarray(x, dtype=np.float64).copy()
    k_new = np.zeros((g.n_layers, nkv, hd))
    v_new = np.zeros((g.n_layers, nkv, hd))
    for l in range(g.n_layers):
        lw = model.layer(l)
        a = rms_norm(x, lw["attn_norm"], g.rms_eps)
        q = rms_norm((lw["wq"] @ a).reshape(nq, hd), lw["q_norm"], g.rms_eps)
        k = rms_norm((lw["wk"] @ a).reshape(nkv, hd), lw["k_norm"], g.rms_eps)
        v = (lw["wv"] @ a).reshape(nkv, hd)
        q = rope(q, pos, g.rope_base)
        k = rope(k, pos, g.rope_base)
        if kv_round:
            k, v = bf16_round(k), bf16_round(v)
        k_new[l], v_new[l] = k, v
        o = np.zeros((nq, hd))
        for h in range(nq):
            kv = kv_head_of(h, nq, nkv)
            keys = np.concatenate([K[l, :pos, kv, :], k[kv][None, :]], axis=0)   # [pos+1, hd]
            vals = np.concatenate([V[l, :pos, kv, :], v[kv][None, :]], axis=0)
            s = (keys @ q[h]) * scale
            s = s - s.max()
            w = np.exp(s)
            o[h] = (w / w.sum()) @ vals
        x = x + lw["wo"] @ o.reshape(nq * hd)
        m = rms_norm(x, lw["ffn_norm"], g.rms_eps)
        x = x + lw["w_down"] @ (silu(lw["w_gate"] @ m) * (lw["w_up"] @ m))
    H = rms_norm(x, model.output_norm, g.rms_eps)
    logits = model.head @ H
    assert np.all(np.isfinite(logits))
    srt = np.sort(logits)
    return {"H": H, "logits": logits, "q0": int(argmax_lowest(logits)),
            "margin": float(srt[-1] - srt[-2]), "k_new": k_new, "v_new": v_new}


def run_steps(model: TalkerOracle, X: np.ndarray, pos0: int, K: np.ndarray, V: np.ndarray,
              kv_round: bool = True) -> List[Dict[str, np.ndarray]]:
    """Consecutive decode steps of one request: X [n, d] at positions
    pos0 .. pos0+n-1 over a history K, V [L, >= pos0, nkv, hd]; the cache
    grows by one position per step."""
    g = model.g
    n = X.shape[0]
    Kc = np.zeros((g.n_layers, pos0 + n, g.n_kv_heads, g.head_dim))
    Vc = np.zeros_like(Kc)
    Kc[:, :pos0], Vc[:, :pos0] = K[:, :pos0], V[:, :pos0]
    out = []
    for i in range(n):
        r = decode_step(model, X[i], pos0 + i, Kc, Vc, kv_round)
        Kc[:, pos0 + i], Vc[:, pos0 + i] = r["k_new"], r["v_new"]
        out.append(r)
    return out


def forward_full(model: TalkerOracle, X: np.ndarray, kv_round: bool = True) -> np.ndarray:
    """Brute force, no cache: the whole sequence X [T, d] (positions 0..T-1)
    through the stack with explicit loops and an explicit causal mask, the
    keys and values rounded as the cache stores them.  Returns H [T, d]."""
    g = model.g
    T = X.shape[0]
    hd, nq, nkv = g.head_dim, g.n_q_heads, g.n_kv_heads
    x = np.asarray(X, dtype=np.float64).copy()
    for l in range(g.n_layers):
        lw = model.layer(l)
        a = rms_norm(x, lw["attn_norm"], g.rms_eps)
        q = rms_norm((a @ lw["wq"].T).reshape(T, nq, hd), lw["q_norm"], g.rms_eps)
        k = rms_norm((a @ lw["wk"].T).reshape(T, nkv, hd), lw["k_norm"], g.rms_eps)
        v = (a @ lw["wv"].T).reshape(T, nkv, hd)
        for t in range(T):
            q[t] = rope(q[t], t, g.rope_base)
            k[t] = rope(k[t], t, g.rope_base)
        if kv_round:
            k, v = bf16_round(k), bf16_round(v)
        o = np.zeros((T, nq, hd))
        for h in range(nq):
            kv = kv_head_of(h, nq, nkv)
            for t in range(T):
                scores = []
                for u in range(T):
                    if u <= t:                       # causal mask
                        scores.append(sum(q[t, h, d] * k[u, kv, d] for d in range(hd)) / math.sqrt(hd))
                mx = max(scores)
                w = [math.exp(s_ - mx) for s_ in scores]
                tot = sum(w)
                for u in range(t + 1):
                    o[t, h] += (w[u] / tot) * v[u, kv]
        x = x + o.reshape(T, nq * hd) @ lw["wo"].T
        m = rms_norm(x, lw["ffn_norm"], g.rms_eps)
        x = x + (silu(m @ lw["w_gate"].T) * (m @ lw["w_up"].T)) @ lw["w_down"].T
    return rms_norm(x, model.output_norm, g.rms_eps)
