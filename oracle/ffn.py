"""Grouped expert FFN + top-k blend oracle, float64.

Test infrastructure only (see the package docstring).

What is computed, restated from the pages:

* metrale ``fp8_moe_grouped.rs``, doc of ``moe_expert_gate_up_act_fp8_grouped``:
  for every active expert, each row routed to it gets ``silu(gate) * up`` of
  the expert's gate and up projections of that row's activations; doc of
  ``moe_expert_down_act_fp8_grouped``: the down projection of that product;
  rows of these intermediates are sorted positions, while the shared expert's
  rows are tokens.  The shared expert is applied to every token.
* nbxtensor ``moe_decode_vec.py``: SwiGLU is ``g * sigmoid(g) * u``
  (the gate/up kernel's epilogue comment); the top-k partials are combined by
  the router weights in a fixed order (``moe_part_reduce_kernel`` docstring).
* metrale ``fp8_moe_grouped.rs``, doc of ``moe_weighted_sum_blend_fp8_grouped``:
  a token's output is the router-weighted sum of its slots' expert outputs,
  each looked up through ``token_to_perm[token*top_k + k]``, plus the shared
  expert's output (ungated when no gate weight is given).
* ``fp8_grouped_tc_shape_ok`` doc: FP8 projections come in whole 128 blocks,
  the FP8 scale blocks.  Reading: one float32 scale per 128x128 block of the
  row-major ``[N, K]`` matrix, and a weight's value is its e4m3 value times the
  block's scale.

Everything is float64 with no intermediate rounding: activations and weights
are widened exactly, products and sums are float64, so the oracle is the exact
result up to float64 rounding.  Slots whose id is outside ``[0, E)`` are
skipped and add nothing to the blend (the align's bounds check).
"""

from __future__ import annotations

from typing import Callable, Iterable, Optional

import numpy as np

from .align import align
from .numerics import bf16_to_f64, e4m3_decode, mxfp4_decode

FP8_BLOCK = 128


def dequant(bits: np.ndarray, scales: Optional[np.ndarray], wdt: str) -> np.ndarray:
    """Weight matrix [N, K] as float64.  bf16: exact widening.  fp8: e4m3 value
    of each code times the float32 scale of its 128x128 block.  fp8_rows: e4m3
    value times the float32 scale of its row (the FP8 page's shared-expert
    weights carry a row scale beside the codes, where the routed experts carry
    128x128 block scales).  mxfp4: packed E2M1 codes [N, K/2] times the E8M0
    scale of each row's 32-column block (``mxfp4_decode``)."""
    if wdt == "bf16":
        return bf16_to_f64(bits)
    if wdt == "fp8_rows":
        vals = e4m3_decode(bits)
        s = np.asarray(scales, dtype=np.float32).astype(np.float64)
        assert s.shape == (vals.shape[0],)
        return vals * s[:, None]
    if wdt == "mxfp4":
        return mxfp4_decode(bits, scales)
    if wdt != "fp8":
        raise ValueError(wdt)
    vals = e4m3_decode(bits)
    N, K = vals.shape
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    assert s.shape == (N // FP8_BLOCK, K // FP8_BLOCK)
    # block (r // 128, c // 128) scales element (r, c)
    return vals * np.repeat(np.repeat(s, FP8_BLOCK, axis=0), FP8_BLOCK, axis=1)


def silu(g: np.ndarray) -> np.ndarray:
    """SiLU: g * sigmoid(g) = g / (1 + exp(-g))."""
    return g / (1.0 + np.exp(-g))


def expert_ffn(x_rows: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray):
    """One expert over its rows.  x_rows [r, H]; Wg, Wu [I, H]; Wd [H, I].
    Returns (act [r, I] = silu(x Wg^T) * (x Wu^T), y [r, H] = act Wd^T)."""
    g = x_rows @ Wg.T
    u = x_rows @ Wu.T
    act = silu(g) * u
    return act, act @ Wd.T


def shared_gate(x_bits: np.ndarray, gate_bits: np.ndarray) -> np.ndarray:
    """Gate of the shared expert per token: sigmoid(x[t] . g), float64.

    The FP8 page's blend takes the layer input and the shared expert's gate
    weight (a hidden-sized vector) beside the shared output, and runs ungated
    when no gate weight is given; it does not print the formula.  Reading: the
    shared output is scaled by the logistic sigmoid of the input's dot product
    with the gate weight."""
    x = bf16_to_f64(x_bits)
    g = bf16_to_f64(np.asarray(gate_bits).reshape(-1))
    return 1.0 / (1.0 + np.exp(-(x @ g)))


def blend(expert_out, topk_weights: np.ndarray, token_to_perm: np.ndarray,
          sh_out: Optional[np.ndarray], tokens: Optional[Iterable[int]] = None,
          H: Optional[int] = None, sh_gate: Optional[np.ndarray] = None) -> np.ndarray:
    """out[t] = sum_k w[t, k] * expert_out[token_to_perm[t*top_k + k]]
    (+ sh_out[t], times sh_gate[t] when a gate is given).

    ``expert_out`` is indexed by sorted position (an array or a dict of rows);
    a slot with ``token_to_perm == -1`` contributes nothing; ``sh_gate`` holds
    one float64 gate per token (all M tokens).  Returns float64 rows for
    ``tokens`` (all tokens by default)."""
    w = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    M, top_k = w.shape
    tokens = list(range(M)) if tokens is None else list(tokens)
    if H is None:
        if sh_out is not None:
            H = sh_out.shape[1]
        elif isinstance(expert_out, dict):
            H = len(next(iter(expert_out.values())))
        else:
            H = np.asarray(expert_out).shape[1]
    out = np.zeros((len(tokens), H), dtype=np.float64)
    for r, t in enumerate(tokens):
        acc = np.zeros(H, dtype=np.float64)
        for k in range(top_k):
            pos = int(token_to_perm[t * top_k + k])
            if pos < 0:
                continue
            acc = acc + w[t, k] * np.asarray(expert_out[pos], dtype=np.float64)
        if sh_out is not None:
            acc = acc + (sh_out[t] if sh_gate is None else sh_gate[t] * sh_out[t])
        out[r] = acc
    return out


def moe_layer(x_bits: np.ndarray, topk_ids: np.ndarray, topk_weights: np.ndarray,
              E: int, BS: int, wdt: str,
              routed_weight: Callable, shared_weight: Optional[Callable] = None,
              tokens: Optional[Iterable[int]] = None, sh_gate_bits: Optional[np.ndarray] = None) -> dict:
    """The whole layer for ``tokens`` (default: all).

    ``routed_weight(which, e)`` and ``shared_weight(which)`` return the raw
    ``(bits, scales)`` of matrix ``which`` in {"gate", "up", "down"};
    ``shared_weight`` is None when there is no shared expert;
    ``sh_gate_bits`` (bf16 [H]) gates it, ``shared_gate``.

    Expert by expert (each expert's weights are dequantised once): the rows
    routed to it are the slots with its id, in ascending flat index, and a
    slot ``i``'s activation row is token ``i // top_k``.

    Returns ``out`` [len(tokens), H] float64 plus the intermediates keyed the
    way the grouped path lays them out: ``act_pos`` / ``y_pos`` (dicts from
    sorted position to row), ``sh_act`` / ``sh_out`` (rows of ``tokens``), and
    the alignment ``tables``.
    """
    ids = np.asarray(topk_ids).astype(np.int64)
    M, top_k = ids.shape
    flat = ids.reshape(-1)
    x = bf16_to_f64(x_bits)
    H = x.shape[1]
    tokens = list(range(M)) if tokens is None else list(tokens)
    tables = align(ids, E, BS)
    perm = tables["token_to_perm"]

    wanted = [t * top_k + k for t in tokens for k in range(top_k)]
    by_expert = {}
    for i in wanted:
        e = int(flat[i])
        if 0 <= e < E:
            by_expert.setdefault(e, []).append(i)

    act_pos, y_pos = {}, {}
    for e in sorted(by_expert):
        slots = sorted(by_expert[e])
        Wg = dequant(*routed_weight("gate", e), wdt)
        Wu = dequant(*routed_weight("up", e), wdt)
        Wd = dequant(*routed_weight("down", e), wdt)
        act, y = expert_ffn(x[[i // top_k for i in slots]], Wg, Wu, Wd)
        for r, i in enumerate(slots):
            act_pos[int(perm[i])] = act[r]
            y_pos[int(perm[i])] = y[r]

    sh_act = sh_out = None
    if shared_weight is not None:
        Wg = dequant(*shared_weight("gate"), wdt)
        Wu = dequant(*shared_weight("up"), wdt)
        Wd = dequant(*shared_weight("down"), wdt)
        sh_act, sh_out = expert_ffn(x[tokens], Wg, Wu, Wd)

    sh_full = None
    if sh_out is not None:
        sh_full = np.zeros((M, H), dtype=np.float64)
        sh_full[tokens] = sh_out
    gate = None if (sh_gate_bits is None or sh_out is None) else shared_gate(x_bits, sh_gate_bits)
    out = blend(y_pos, topk_weights, perm, sh_full, tokens=tokens, H=H, sh_gate=gate)
    return {"out": out, "act_pos": act_pos, "y_pos": y_pos, "sh_act": sh_act,
            "sh_out": sh_out, "tables": tables, "tokens": tokens}
