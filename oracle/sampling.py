"""Caller-controlled sampling of a codebook token from one step's logits.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the GPU library and never calls it.

The pages describe the exported predictor as greedy (mixtureofinsights
OpenVINO port, section 2.2) and leave sampling to the caller: the GGUF
loaders do not read the generation config, and how to sample is the caller's
choice (rightkit-qts exporter README, "Qwen3-TTS 1.7B -> QTS GGUF", section
"Usage").  What a caller usually controls when it samples (temperature,
top-k, top-p) is taken here in its plainest form.  Every tie and rounding
decision is fixed, so that two implementations can be compared token by
token.  For one request and one step, with logits z over the vocabulary:

1. Rank order: descending logit, and the lower vocabulary index first among
   equal logits.  The logits are ranked as fp32 values, the precision the
   GPU decides in.
2. Temperature T > 0: rank r gets the weight w_r = exp((z_r - z_0) / T),
   where z_0 is the largest logit.  Subtracting z_0 changes no probability.
3. Top-k: keep the ranks r < K, exactly K tokens; K = 0 (or K >= V) keeps
   every token.
4. Top-p: among the tokens kept so far, keep the shortest rank-order prefix
   whose weight reaches P times their total weight (at least one token).
   P = 1 keeps them all.
5. Draw: the caller supplies one uniform u per request and step.  It is
   clamped to [0, 1], and NaN counts as 0.  The token is the first kept rank
   whose inclusive cumulative weight exceeds u times the final kept total, or
   the last kept rank if none does (u = 1).

This is inverse-CDF sampling from softmax(z / T) restricted to the kept set.
Any u in [0, 1) maps to one token, and token r owns an interval of u whose
length is its renormalised probability.

The arithmetic here is float64 on the fp32-rounded logits and uniforms.  The
GPU sums in fp32, in its own order.  A decision therefore counts as unique
only when both thresholds (u times the total for the draw, P times the total
for the top-p cut) lie farther than a stated relative margin from every
cumulative boundary.  ``sample_token`` returns that margin.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np


def rank_order(z: np.ndarray) -> np.ndarray:
    """Vocabulary indices by descending fp32 logit, lower index first on ties."""
    z32 = np.asarray(z, dtype=np.float32).astype(np.float64)
    idx = np.arange(z32.shape[0])
    # lexsort sorts by the last key first: primary -z (descending), then index
    return np.lexsort((idx, -z32))


def clamp_uniform(u: float) -> float:
    u = float(np.float32(u))
    if math.isnan(u):
        return 0.0
    return min(max(u, 0.0), 1.0)


def explain(z: np.ndarray, temperature: float, top_k: int, top_p: float, u: float) -> dict:
    """Every intermediate of one draw (module header, steps 1-5): the rank
    order, the cumulative weights c1 of the top-k ranks and their total s1,
    the kept count n2 after top-p, the kept total s2, the draw threshold
    u * s2 and the drawn rank."""
    assert temperature > 0.0 and math.isfinite(temperature)
    assert 0.0 < top_p <= 1.0
    assert top_k >= 0
    z32 = np.asarray(z, dtype=np.float32).astype(np.float64)
    V = z32.shape[0]
    order = rank_order(z32)
    zs = z32[order]
    w = np.exp((zs - zs[0]) / float(np.float32(temperature)))
    n1 = V if (top_k == 0 or top_k >= V) else top_k
    c1 = np.cumsum(w[:n1])
    s1 = c1[-1]
    cut = None
    if top_p >= 1.0:
        n2 = n1
    else:
        cut = float(np.float32(top_p)) * s1
        reach = np.nonzero(c1 >= cut)[0]
        n2 = int(reach[0]) + 1 if reach.size else n1
    s2 = c1[n2 - 1]
    thr = clamp_uniform(u) * s2
    above = np.nonzero(c1[:n2] > thr)[0]
    rank = int(above[0]) if above.size else n2 - 1
    return {"order": order, "c1": c1, "s1": s1, "cut": cut, "n2": n2, "s2": s2, "thr": thr, "rank": rank}


def sample_token(z: np.ndarray, temperature: float, top_k: int, top_p: float,
                 u: float) -> Tuple[int, float, int]:
    """One token from logits z (length V) under the steps of the module header.

    Returns (token, margin, kept): the vocabulary index drawn; the smallest
    relative distance, as a fraction of the relevant total, between a
    threshold and a cumulative boundary; and the number of tokens kept after
    top-k and top-p."""
    e = explain(z, temperature, top_k, top_p, u)
    c1, n2 = e["c1"], e["n2"]
    margin = math.inf
    if e["cut"] is not None:
        margin = min(margin, float(np.min(np.abs(c1 - e["cut"]))) / e["s1"])
    # distance to the interior boundaries (the last one is s2 itself, which
    # only u = 1 reaches, and that draws the last kept rank either way)
    inner = c1[: n2 - 1]
    if inner.size:
        margin = min(margin, float(np.min(np.abs(inner - e["thr"]))) / e["s2"])
    return int(e["order"][e["rank"]]), margin, n2


def sample_rows(logits: np.ndarray, temperature: float, top_k: int, top_p: float,
                uniforms: np.ndarray):
    """sample_token over the rows of logits [N, V] with uniforms [N].
    Returns tokens [N] int64 and margins [N]."""
    logits = np.asarray(logits)
    N = logits.shape[0]
    tok = np.zeros(N, dtype=np.int64)
    mar = np.zeros(N)
    for i in range(N):
        tok[i], mar[i], _ = sample_token(logits[i], temperature, top_k, top_p, uniforms[i])
    return tok, mar
