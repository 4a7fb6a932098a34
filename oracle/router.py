"""Per-row router oracle, float64: the step before the path.

Test infrastructure only (see the package docstring).

What is computed, restated from the pages:

* metrale ``forward_nvfp4_grouped_decode.rs`` source page: the decode layer's
  admission predicate requires the per-row router (a BF16 softmax gate with no
  correction bias, fed the already-normalised input) and its two kernels, a
  router GEMV over the batch rows and a per-row top-k softmax; the layer then
  routes each row (``grouped_route`` with per-row routing) into per-slot expert
  indices and float32 weights.
* The workload recipe the path is measured on: softmax over the experts, top-k,
  weights renormalised over the k chosen.

Readings (the pages show neither kernel's source):

* logits[t, e] = sum_h W[e, h] * x[t, h] with W the bf16 gate weight [E, H];
* the k chosen experts are the k largest logits, larger first, equal logits in
  ascending expert order (the order a stable descending sort gives);
* a chosen expert's weight is its softmax probability divided by the sum of the
  chosen probabilities, which is the softmax taken over the chosen logits alone
  (the full softmax's denominator cancels).
"""

from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f64


def router_logits(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """float64 logits [M, E] of bf16 activations [M, H] and bf16 gate weight
    [E, H] (both as uint16 bits): every product and sum in float64."""
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    return x @ w.T


def topk_softmax(logits: np.ndarray, top_k: int):
    """(ids int64 [M, top_k], weights float64 [M, top_k]) from logits [M, E]:
    per row the top_k largest logits (larger first, ties to the lower expert)
    and the softmax over the chosen logits."""
    logits = np.asarray(logits, dtype=np.float64)
    M, E = logits.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k must be in [1, E]")
    ids = np.empty((M, top_k), dtype=np.int64)
    wts = np.empty((M, top_k), dtype=np.float64)
    for t in range(M):
        row = logits[t]
        order = sorted(range(E), key=lambda e: (-row[e], e))[:top_k]
        chosen = row[order]
        p = np.exp(chosen - chosen[0])
        ids[t] = order
        wts[t] = p / p.sum()
    return ids, wts
