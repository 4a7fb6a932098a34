"""Seeded generators for the five workload shapes of the MoE layer.

Recipe (each choice is a reading of the workload descriptions; the reasons
are recorded in the design notes):

* activations ``x``: bf16 bits of N(0, 1) float32 draws, round-to-nearest-even;
* router output: softmax over N(0, 1) fp64 logits (plus a per-expert N(0, std)
  bias for the skewed verify workload), top-k by a stable sort of the
  probabilities (ties go to the lower expert), the k weights renormalised to
  sum to one and stored float32; the align-only workload draws ids from a
  finite Zipf law over a seeded permutation of the experts, distinct within a
  token, with equal weights 1/top_k;
* bf16 expert weights: N(0, 0.02) float32 draws rounded to bf16;
* fp8 expert weights: U(-1/sqrt(K), 1/sqrt(K)) float32 draws for a K-deep
  matrix, one float32 scale per 128x128 block equal to the block's absolute
  maximum over 448 (1 for an all-zero block), codes = OCP e4m3fn of
  ``w / scale`` rounded to nearest even (torch's float8_e4m3fn cast);
* mxfp4 expert weights: the same draws, OCP microscaling quantisation (E2M1
  codes, one E8M0 scale per 32 columns of a row, see ``_draw_mxfp4``).

Weight matrices are row-major ``[N, K]`` (output rows, input columns): gate and
up are ``[I, H]``, down is ``[H, I]``; a shared expert uses ``S`` for ``I``.
"""

from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Callable, Optional, Tuple

import numpy as np

FP8_BLOCK = 128

# purpose tags of the PCG64 streams ([seed, tag, index])
_TAG_X = 1
_TAG_LOGITS = 2
_TAG_BIAS = 3
_TAG_ZIPF_PERM = 4
_TAG_ZIPF_DRAW = 5
_TAG_ROUTED = {"gate": 10, "up": 11, "down": 12}
_TAG_SHARED = {"gate": 20, "up": 21, "down": 22}
_TAG_ROUTER = 30
_TAG_SHARED_GATE = 31


@dataclass(frozen=True)
class MoeConfig:
    name: str
    M: int          # tokens (rows)
    H: int          # hidden size
    E: int          # routed experts
    top_k: int
    I: int          # routed expert intermediate size
    S: int          # shared expert intermediate size (0: no shared expert)
    BS: int         # alignment block size
    wdt: Optional[str]      # "bf16" | "fp8" (128x128 block scales) | "fp8_rows" (row scales) | None
    routing: str            # "softmax" | "softmax_bias" | "zipf"
    bias_std: float = 0.0
    zipf_s: float = 0.0
    seed: int = 0

    @property
    def n(self) -> int:
        return self.M * self.top_k

    @property
    def has_ffn(self) -> bool:
        return self.wdt is not None

    def replace(self, **kw) -> "MoeConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # M=4, hidden 256, 8 experts, top-2, inter 128, BS 16, bf16 weights N(0, 0.02)
    "tiny": MoeConfig("tiny", 4, 256, 8, 2, 128, 0, 16, "bf16", "softmax", seed=1001),
    # M=8, hidden 2048, 128 experts, top-8, inter 768, BS 16, fp8 block-scaled, no shared expert
    "decode": MoeConfig("decode", 8, 2048, 128, 8, 768, 0, 16, "fp8", "softmax", seed=1002),
    # M=128, as decode plus an always-on shared expert of inter 2048; logits biased per expert
    "verify": MoeConfig("verify", 128, 2048, 128, 8, 768, 2048, 16, "fp8", "softmax_bias",
                        bias_std=2.0, seed=1003),
    # align only: M=4096, 256 experts, top-8, BS 64, Zipf(1.1) ids distinct within a token
    "align": MoeConfig("align", 4096, 0, 256, 8, 0, 0, 64, None, "zipf", zipf_s=1.1, seed=1004),
    # M=64, hidden 7168, 256 experts, top-8, inter 2048, shared inter 2048, BS 64, fp8
    "large": MoeConfig("large", 64, 7168, 256, 8, 2048, 2048, 64, "fp8", "softmax", seed=1005),
}


def _rng(cfg: MoeConfig, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([cfg.seed, tag, index])


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits.
    Inputs here are finite draws, so no NaN handling is needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def x_bf16(cfg: MoeConfig) -> np.ndarray:
    """Activations [M, H] as bf16 bits (uint16)."""
    z = _rng(cfg, _TAG_X).standard_normal((cfg.M, cfg.H), dtype=np.float32)
    return bf16_bits_from_f32(z)


def routing(cfg: MoeConfig) -> Tuple[np.ndarray, np.ndarray]:
    """Router output: (topk_ids int64 [M, top_k], topk_weights float32 [M, top_k])."""
    M, E, k = cfg.M, cfg.E, cfg.top_k
    if cfg.routing == "zipf":
        ranks_p = np.arange(1, E + 1, dtype=np.float64) ** (-cfg.zipf_s)
        ranks_p /= ranks_p.sum()
        perm = _rng(cfg, _TAG_ZIPF_PERM).permutation(E)
        draw = _rng(cfg, _TAG_ZIPF_DRAW)
        ids = np.empty((M, k), dtype=np.int64)
        for t in range(M):
            ids[t] = perm[draw.choice(E, size=k, replace=False, p=ranks_p)]
        w = np.full((M, k), 1.0 / k, dtype=np.float32)
        return ids, w
    logits = _rng(cfg, _TAG_LOGITS).standard_normal((M, E))
    if cfg.routing == "softmax_bias":
        logits = logits + _rng(cfg, _TAG_BIAS).normal(0.0, cfg.bias_std, size=E)[None, :]
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    ids = np.argsort(-p, axis=1, kind="stable")[:, :k].astype(np.int64)
    w = np.take_along_axis(p, ids, axis=1)
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def router_weight_bf16(cfg: MoeConfig) -> np.ndarray:
    """Router gate weight [E, H] as bf16 bits, N(0, 1/H): with N(0, 1)
    activations the logits come out near N(0, 1), like the routing recipe's."""
    z = _rng(cfg, _TAG_ROUTER).normal(0.0, 1.0 / np.sqrt(cfg.H), size=(cfg.E, cfg.H)).astype(np.float32)
    return bf16_bits_from_f32(z)


def shared_gate_bf16(cfg: MoeConfig) -> np.ndarray:
    """Gate vector of the shared expert's output [H] as bf16 bits, N(0, 1/H):
    with N(0, 1) activations its dot products come out near N(0, 1)."""
    z = _rng(cfg, _TAG_SHARED_GATE).normal(0.0, 1.0 / np.sqrt(cfg.H), size=cfg.H).astype(np.float32)
    return bf16_bits_from_f32(z)


def weight_shape(cfg: MoeConfig, which: str, shared: bool = False) -> Tuple[int, int]:
    inter = cfg.S if shared else cfg.I
    if which in ("gate", "up"):
        return inter, cfg.H
    if which == "down":
        return cfg.H, inter
    raise ValueError(which)


def _draw_matrix(cfg: MoeConfig, rng: np.random.Generator, N: int, K: int):
    if cfg.wdt == "bf16":
        w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
        return bf16_bits_from_f32(w), None
    if cfg.wdt == "mxfp4":
        return _draw_mxfp4(rng, N, K)
    if cfg.wdt not in ("fp8", "fp8_rows"):
        raise ValueError(f"config {cfg.name} has no expert weights")
    import torch  # the float8 cast is torch's; it is the only use of torch here

    if N % FP8_BLOCK or K % FP8_BLOCK:
        raise ValueError("fp8 weights need N and K in whole 128 blocks")
    a = np.float32(1.0 / np.sqrt(K))
    w = (rng.random((N, K), dtype=np.float32) * np.float32(2.0) - np.float32(1.0)) * a
    if cfg.wdt == "fp8_rows":  # one float32 scale per row: row amax / 448
        amax = np.abs(w).max(axis=1)
        scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
        q = np.clip(w / scale[:, None], -448.0, 448.0)
        codes = torch.from_numpy(np.ascontiguousarray(q)).to(torch.float8_e4m3fn)
        return codes.view(torch.uint8).numpy().copy(), scale
    nb, kb = N // FP8_BLOCK, K // FP8_BLOCK
    blocks = w.reshape(nb, FP8_BLOCK, kb, FP8_BLOCK)
    amax = np.abs(blocks).max(axis=(1, 3))
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = blocks / scale[:, None, :, None]
    q = np.clip(q, -448.0, 448.0).reshape(N, K)
    codes = torch.from_numpy(np.ascontiguousarray(q)).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8).numpy().copy(), scale


# magnitudes of the E2M1 codes 0..7 (codes 8..15 are their negatives)
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
MX_BLOCK = 32


def _draw_mxfp4(rng: np.random.Generator, N: int, K: int):
    """U(-1/sqrt(K), 1/sqrt(K)) draws quantised the OCP microscaling way: per
    32-column block of a row, scale exponent floor(log2(amax)) - 2 (2 is the
    largest E2M1 exponent, so the block's amax lands in [4, 8)); elements
    divided by the scale and rounded to the nearest E2M1 value (ties to the
    even code), saturating at 6.  Returns (packed codes uint8 [N, K/2], lower
    nibble = even column; E8M0 scale bytes uint8 [N, K/32]); an all-zero block
    gets scale byte 127 (1.0)."""
    if N % 128 or K % 128:
        raise ValueError("mxfp4 weights need N and K in whole 128 blocks")
    a = np.float32(1.0 / np.sqrt(K))
    w = ((rng.random((N, K), dtype=np.float32) * np.float32(2.0) - np.float32(1.0)) * a).astype(np.float64)
    blocks = w.reshape(N, K // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=2)
    exp = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, 0).astype(np.int64)
    exp = np.clip(exp, -127, 127)
    q = np.abs(blocks) / np.exp2(exp)[:, :, None]
    # nearest magnitude, ties to the even code
    idx = np.searchsorted(_E2M1_MAG, q)  # first magnitude >= q
    idx = np.clip(idx, 1, 7)
    lo, hi = _E2M1_MAG[idx - 1], _E2M1_MAG[idx]
    pick_hi = (q - lo > hi - q) | ((q - lo == hi - q) & (idx % 2 == 0))
    code = np.where(q >= 6.0, 7, np.where(pick_hi, idx, idx - 1)).astype(np.uint8)
    code = code | np.where(blocks < 0, 8, 0).astype(np.uint8)
    code = code.reshape(N, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(packed), (exp + 127).astype(np.uint8)


def expert_matrix(cfg: MoeConfig, which: str, e: int):
    """Routed expert ``e``'s ``which`` matrix: (bits [N, K], scales [N/128, K/128] or None).
    bf16 weights come as uint16 bits, fp8 weights as uint8 e4m3fn codes (row
    scales [N] for fp8_rows), mxfp4 weights as packed uint8 codes [N, K/2] with
    E8M0 scale bytes [N, K/32]."""
    N, K = weight_shape(cfg, which)
    return _draw_matrix(cfg, _rng(cfg, _TAG_ROUTED[which], e), N, K)


def shared_matrix(cfg: MoeConfig, which: str):
    """The shared expert's ``which`` matrix, or None when the config has none."""
    if cfg.S == 0:
        return None
    N, K = weight_shape(cfg, which, shared=True)
    return _draw_matrix(cfg, _rng(cfg, _TAG_SHARED[which], 0), N, K)


def fill_expert_weights(cfg: MoeConfig, which: str, sink: Callable, threads: int = 8,
                        experts=None) -> None:
    """Draw every routed expert's ``which`` matrix (in parallel) and hand each to
    ``sink(e, bits, scales)``; ``sink`` may be called from worker threads."""
    experts = range(cfg.E) if experts is None else experts

    def one(e):
        bits, sc = expert_matrix(cfg, which, e)
        sink(e, bits, sc)

    if threads <= 1:
        for e in experts:
            one(e)
        return
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, experts))
