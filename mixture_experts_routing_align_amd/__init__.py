"""MI355X (gfx950) MoE routing-align + grouped expert FFN.

Thin Python binding of ``libmoe_mi355x.so`` (C ABI in ``include/moe_mi355x.h``).
Every function here only marshals arguments: torch tensors supply device
memory and the current HIP stream, and each step runs in the library's HIP
kernels.  There is no fallback: if the library is not built, importing the
binding's entry points raises.

Entry points (same names as the C ABI): ``moe_align``,
``moe_grouped_gate_up_silu``, ``moe_grouped_down``, ``moe_blend``,
``moe_layer_forward`` (via :class:`MoeLayer`), ``moe_layer_workspace_bytes``,
``moe_align_max_total``, ``moe_active_cap``, ``moe_tile_weights``,
``moe_tiled_weight_bytes``, ``moe_align_gate_up_silu``.

Weights are passed as ``(w, scale)`` pairs: ``w`` is ``[E, N, K]``
``torch.uint8`` e4m3fn codes with ``scale`` float32 ``[E, N/128, K/128]`` (one
per 128x128 block) or ``[E, N]`` (one per row), or ``[E, N, K/2]``
``torch.uint8`` MXFP4 codes (two E2M1 codes per byte, lower nibble first) with
``scale`` ``torch.uint8`` E8M0 ``[E, N, K/32]``, or ``torch.bfloat16`` with
``scale`` None - or as the :class:`TiledWeight` that ``moe_tile_weights`` makes
from such a pair.  A shared expert's ``[N, K]`` matrix takes ``[N/128, K/128]``
or ``[N]`` scales (MXFP4: ``[N, K/2]`` codes, ``[N, K/32]`` scales).
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from . import _ffi
from ._ffi import (  # noqa: F401
    MOE_ERR_HIP,
    MOE_ERR_LIMIT,
    MOE_ERR_NULL,
    MOE_ERR_SHAPE,
    MOE_ERR_WORKSPACE,
    MOE_IDX_I32,
    MOE_IDX_I64,
    MOE_FUSED_ALIGN_MAX_SLOTS,
    MOE_FUSED_LAYER_MAX_SLOTS,
    MOE_LAYER_PATH_AUTO,
    MOE_LAYER_PATH_NARROW,
    MOE_LAYER_PATH_SINGLE_PASS,
    MOE_LAYER_PATH_STEPS,
    MOE_LAYER_WORKSPACE_REGIONS,
    MOE_MAX_EXPERTS,
    MOE_NARROW_AUTO_SLOTS,
    MOE_NARROW_LAYER_MAX_SLOTS,
    MOE_OK,
    MOE_ROUTER_MAX_TOP_K,
    MOE_W_BF16,
    MOE_W_BF16_TILED,
    MOE_W_FP8_E4M3,
    MOE_W_FP8_E4M3_ROWS,
    MOE_W_FP8_E4M3_ROWS_TILED,
    MOE_W_FP8_E4M3_TILED,
    MOE_W_MXFP4,
    MOE_W_MXFP4_TILED,
    TABLE_FIELDS,
    MoeAlignTables,
    MoeLayerDesc,
    MoeWeight,
)

Weight = Tuple[torch.Tensor, Optional[torch.Tensor]]


class MoeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


def lib():
    return _ffi.load()


def _check(rc: int) -> None:
    if rc != MOE_OK:
        raise MoeError(rc, lib().moe_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


# ------------------------------------------------------------------ sizing --

def moe_align_max_total(n: int, E: int, BS: int) -> int:
    return int(lib().moe_align_max_total(n, E, BS))


def moe_active_cap(n: int, E: int) -> int:
    return int(lib().moe_active_cap(n, E))


# ------------------------------------------------------------------- align --

@dataclass
class AlignTables:
    sorted_token_ids: torch.Tensor
    block_expert_ids: torch.Tensor
    expert_offsets: torch.Tensor
    expert_counts: torch.Tensor
    token_to_perm: torch.Tensor
    active_experts: torch.Tensor
    active_count: torch.Tensor
    total: torch.Tensor

    @classmethod
    def allocate(cls, M: int, top_k: int, E: int, BS: int, device="cuda") -> "AlignTables":
        n = M * top_k
        mt = moe_align_max_total(n, E, BS)
        cap = moe_active_cap(n, E)
        _need(mt >= 0 and cap >= 0, "invalid alignment shape")

        def mk(k):
            return torch.empty(k, dtype=torch.int32, device=device)

        return cls(mk(mt), mk(mt // BS), mk(E + 1), mk(E), mk(n), mk(cap), mk(1), mk(1))

    def as_c(self) -> MoeAlignTables:
        return MoeAlignTables(*[getattr(self, f).data_ptr() for f in TABLE_FIELDS])


def moe_align_workspace_bytes(M: int, top_k: int, E: int) -> int:
    """Bytes of workspace moe_align takes for its two-launch form (0: none needed)."""
    return int(lib().moe_align_workspace_bytes(M, top_k, E))


def moe_align(topk_ids: torch.Tensor, E: int, BS: int, tables: Optional[AlignTables] = None,
              stream=None, workspace: Optional[torch.Tensor] = None) -> AlignTables:
    """Align the [M, top_k] ids (int32 or int64, device); returns the tables.
    With `workspace` (a device buffer of at least moe_align_workspace_bytes
    bytes) the C call is moe_align_ws, else moe_align; the tables are the same."""
    _need(topk_ids.dim() == 2 and topk_ids.is_contiguous(), "topk_ids must be a contiguous [M, top_k] tensor")
    _need(topk_ids.dtype in (torch.int32, torch.int64), "topk_ids must be int32 or int64")
    M, top_k = topk_ids.shape
    if tables is None:
        tables = AlignTables.allocate(M, top_k, E, BS, topk_ids.device)
    idt = MOE_IDX_I64 if topk_ids.dtype == torch.int64 else MOE_IDX_I32
    c = tables.as_c()
    if workspace is None:
        _check(lib().moe_align(topk_ids.data_ptr(), idt, M, top_k, E, BS, ctypes.byref(c), _stream(stream)))
    else:
        nbytes = workspace.numel() * workspace.element_size()
        _check(lib().moe_align_ws(topk_ids.data_ptr(), idt, M, top_k, E, BS, ctypes.byref(c), workspace.data_ptr(),
                                  nbytes, _stream(stream)))
    return tables


def moe_align_ws(topk_ids: torch.Tensor, E: int, BS: int, workspace: torch.Tensor,
                 tables: Optional[AlignTables] = None, stream=None) -> AlignTables:
    """moe_align with a workspace for its blocks' counts (two launches instead of three)."""
    return moe_align(topk_ids, E, BS, tables=tables, stream=stream, workspace=workspace)


# ------------------------------------------------------------ grouped FFN --

@dataclass
class TiledWeight:
    """Expert weights in the tiled layout of ``moe_tile_weights`` (flat bytes),
    with the row-major shape they came from and their (unchanged) scales."""
    w: torch.Tensor
    scale: Optional[torch.Tensor]
    wdt: int
    shape: Tuple[int, int, int]


def weight_dtype(w) -> int:
    """The weight dtype of a pair, a tiled weight or a bare tensor; FP8 scales
    with one dimension fewer than the codes are row scales, and byte codes with
    byte scales are MXFP4."""
    s = None
    if isinstance(w, TiledWeight):
        return w.wdt
    if isinstance(w, tuple):
        w, s = w
    if w.dtype == torch.uint8 and s is not None and s.dtype == torch.uint8:
        return MOE_W_MXFP4
    if w.dtype in (torch.uint8, torch.float8_e4m3fn):
        return MOE_W_FP8_E4M3_ROWS if s is not None and s.dim() == w.dim() - 1 else MOE_W_FP8_E4M3
    if w.dtype == torch.bfloat16:
        return MOE_W_BF16
    raise ValueError(f"unsupported weight dtype {w.dtype}")


def weight_shape(wt) -> Tuple[int, int, int]:
    """(E, N, K) of a weight pair or a tiled weight; a single [N, K] matrix (a
    shared expert) counts as E = 1."""
    if isinstance(wt, TiledWeight):
        return tuple(wt.shape)
    shape = tuple(wt[0].shape)
    if weight_dtype(wt) == MOE_W_MXFP4:  # two codes per byte
        shape = shape[:-1] + (2 * shape[-1],)
    return (1,) + shape if len(shape) == 2 else shape


def _weight(wt) -> Optional[MoeWeight]:
    if wt is None:
        return None
    if isinstance(wt, TiledWeight):
        return MoeWeight(wt.w.data_ptr(), _ptr(wt.scale))
    w, s = wt
    _need(w.is_contiguous() and (s is None or s.is_contiguous()), "weights must be contiguous")
    wdt = weight_dtype(wt)
    if wdt in (MOE_W_FP8_E4M3, MOE_W_FP8_E4M3_ROWS):
        _need(s is not None and s.dtype == torch.float32, "FP8 weights need float32 scales")
    return MoeWeight(w.data_ptr(), _ptr(s))


def moe_tiled_weight_bytes(wdt: int, E: int, N: int, K: int) -> int:
    n = int(lib().moe_tiled_weight_bytes(wdt, E, N, K))
    if n == 0:
        raise MoeError(MOE_ERR_SHAPE, lib().moe_last_error().decode())
    return n


def moe_tile_weights(wt: Weight, stream=None) -> TiledWeight:
    """The tiled copy of a row-major ``(w, scale)`` pair (a new device buffer)."""
    w, s = wt
    _need(w.is_contiguous(), "weights must be contiguous")
    wdt = weight_dtype(wt)
    E, N, K = weight_shape(wt)
    dst = torch.empty(moe_tiled_weight_bytes(wdt, E, N, K), dtype=torch.uint8, device=w.device)
    _check(lib().moe_tile_weights(w.data_ptr(), dst.data_ptr(), wdt, E, N, K, _stream(stream)))
    tiled = {MOE_W_FP8_E4M3: MOE_W_FP8_E4M3_TILED, MOE_W_FP8_E4M3_ROWS: MOE_W_FP8_E4M3_ROWS_TILED,
             MOE_W_BF16: MOE_W_BF16_TILED, MOE_W_MXFP4: MOE_W_MXFP4_TILED}[wdt]
    return TiledWeight(dst, s, tiled, (E, N, K))


def _ref(x):
    return None if x is None else ctypes.byref(x)


def _common_dtype(*weights) -> int:
    """The one weight dtype of the given weights (None entries skipped)."""
    kinds = {weight_dtype(w) for w in weights if w is not None}
    _need(len(kinds) == 1, "all weights of a call must share one dtype, layout and scale form")
    return kinds.pop()


def moe_grouped_gate_up_silu(x: torch.Tensor, gate: Weight, up: Weight, tables: AlignTables, act: torch.Tensor,
                             top_k: int, BS: int, sh_gate: Optional[Weight] = None, sh_up: Optional[Weight] = None,
                             sh_act: Optional[torch.Tensor] = None, stream=None) -> None:
    """act[p] = silu(Wg x) * (Wu x) per sorted slot position (+ the shared expert into sh_act)."""
    M, H = x.shape
    E, I, H2 = weight_shape(gate)
    _need(H2 == H and x.dtype == torch.bfloat16, "x must be bf16 [M, H] matching the weights")
    _need(act.dtype == torch.float32 and act.shape[1] == I, "act must be float32 [max_total, I]")
    S = 0 if sh_gate is None else weight_shape(sh_gate)[1]
    c = tables.as_c()
    wdt = _common_dtype(gate, up, sh_gate, sh_up)
    _check(lib().moe_grouped_gate_up_silu(
        x.data_ptr(), wdt, ctypes.byref(_weight(gate)), ctypes.byref(_weight(up)), ctypes.byref(c),
        act.data_ptr(), _ref(_weight(sh_gate)), _ref(_weight(sh_up)), _ptr(sh_act),
        M, H, I, S, E, top_k, BS, _stream(stream)))


def moe_align_gate_up_silu(topk_ids: torch.Tensor, x: torch.Tensor, gate, up, E: int, BS: int, act: torch.Tensor,
                           tables: Optional[AlignTables] = None, sh_gate=None, sh_up=None,
                           sh_act: Optional[torch.Tensor] = None, stream=None) -> AlignTables:
    """moe_align + moe_grouped_gate_up_silu in one launch (n <= MOE_FUSED_ALIGN_MAX_SLOTS)."""
    _need(topk_ids.dim() == 2 and topk_ids.is_contiguous(), "topk_ids must be a contiguous [M, top_k] tensor")
    _need(topk_ids.dtype in (torch.int32, torch.int64), "topk_ids must be int32 or int64")
    M, top_k = topk_ids.shape
    H = x.shape[1]
    E2, I, H2 = weight_shape(gate)
    _need(E2 == E and H2 == H and x.dtype == torch.bfloat16, "x must be bf16 [M, H] matching the weights")
    _need(act.dtype == torch.float32 and act.shape[1] == I, "act must be float32 [max_total, I]")
    if tables is None:
        tables = AlignTables.allocate(M, top_k, E, BS, topk_ids.device)
    S = 0 if sh_gate is None else weight_shape(sh_gate)[1]
    idt = MOE_IDX_I64 if topk_ids.dtype == torch.int64 else MOE_IDX_I32
    c = tables.as_c()
    _check(lib().moe_align_gate_up_silu(
        topk_ids.data_ptr(), idt, x.data_ptr(), _common_dtype(gate, up, sh_gate, sh_up), ctypes.byref(_weight(gate)),
        ctypes.byref(_weight(up)), ctypes.byref(c), act.data_ptr(), _ref(_weight(sh_gate)), _ref(_weight(sh_up)),
        _ptr(sh_act), M, H, I, S, E, top_k, BS, _stream(stream)))
    return tables


def moe_grouped_down(act: torch.Tensor, down: Weight, tables: AlignTables, expert_out: torch.Tensor, M: int,
                     top_k: int, BS: int, sh_down: Optional[Weight] = None, sh_act: Optional[torch.Tensor] = None,
                     sh_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """expert_out[p] = Wd act[p] per sorted slot position (+ the shared expert into sh_out)."""
    E, H, I = weight_shape(down)
    _need(act.dtype == torch.float32 and act.shape[1] == I, "act must be float32 [max_total, I]")
    _need(expert_out.dtype == torch.float32 and expert_out.shape[1] == H, "expert_out must be float32 [max_total, H]")
    S = 0 if sh_down is None else weight_shape(sh_down)[2]
    c = tables.as_c()
    _check(lib().moe_grouped_down(
        act.data_ptr(), _common_dtype(down, sh_down), ctypes.byref(_weight(down)), ctypes.byref(c),
        expert_out.data_ptr(), _ref(_weight(sh_down)), _ptr(sh_act), _ptr(sh_out),
        M, H, I, S, E, top_k, BS, _stream(stream)))


def moe_blend(out: torch.Tensor, expert_out: torch.Tensor, topk_weights: torch.Tensor, token_to_perm: torch.Tensor,
              sh_out: Optional[torch.Tensor] = None, stream=None, x: Optional[torch.Tensor] = None,
              sh_expert_gate: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[t] = bf16(sum_k w[t,k] expert_out[token_to_perm[t*top_k+k]] + g_t sh_out[t]),
    g_t = sigmoid(x[t] . sh_expert_gate) when a gate vector is given, else 1."""
    M, top_k = topk_weights.shape
    H = out.shape[1]
    _need(out.dtype == torch.bfloat16 and out.shape[0] == M, "out must be bf16 [M, H]")
    _need(topk_weights.dtype == torch.float32 and topk_weights.is_contiguous(), "topk_weights must be float32")
    _need(token_to_perm.dtype == torch.int32, "token_to_perm must be int32")
    _check(lib().moe_blend(out.data_ptr(), expert_out.data_ptr(), topk_weights.data_ptr(), token_to_perm.data_ptr(),
                           _ptr(sh_out), _ptr(x), _ptr(sh_expert_gate), M, H, top_k, _stream(stream)))
    return out


# ------------------------------------------------------------- whole layer --

WORKSPACE_REGIONS = TABLE_FIELDS + ("act", "expert_out", "sh_act", "sh_out", "part", "sh_part")


class MoeLayer:
    """Expert weights of one MoE layer plus the fused ``moe_layer_forward`` call."""

    def __init__(self, gate, up, down, top_k: int, BS: int, sh_gate=None, sh_up=None, sh_down=None,
                 sh_expert_gate: Optional[torch.Tensor] = None, path: int = MOE_LAYER_PATH_AUTO):
        self.gate, self.up, self.down = gate, up, down
        # the path the descriptor asks for (MOE_LAYER_PATH_AUTO: chosen from the shapes)
        self.path_request = path
        self.sh_gate, self.sh_up, self.sh_down = sh_gate, sh_up, sh_down
        # bf16 [H] gate vector of the shared expert's output (None: ungated)
        self.sh_expert_gate = sh_expert_gate
        self.top_k, self.BS = top_k, BS
        self.E, self.I, self.H = weight_shape(gate)
        self.S = 0 if sh_gate is None else weight_shape(sh_gate)[1]
        self.wdt = weight_dtype(gate)
        kinds = {weight_dtype(w) for w in (gate, up, down, sh_gate, sh_up, sh_down) if w is not None}
        _need(len(kinds) == 1, "all weights of a layer must share one dtype and layout")
        self._keep = None

    def tiled(self, stream=None) -> "MoeLayer":
        """The same layer with every weight in the tiled layout."""
        def t(w):
            return None if w is None or isinstance(w, TiledWeight) else moe_tile_weights(w, stream)

        return MoeLayer(t(self.gate), t(self.up), t(self.down), self.top_k, self.BS,
                        t(self.sh_gate), t(self.sh_up), t(self.sh_down), self.sh_expert_gate, self.path_request)

    def with_path(self, path: int) -> "MoeLayer":
        """The same weights with the descriptor asking for `path` (a
        MOE_LAYER_PATH_* value; AUTO lets the library choose)."""
        return MoeLayer(self.gate, self.up, self.down, self.top_k, self.BS, self.sh_gate, self.sh_up, self.sh_down,
                        self.sh_expert_gate, path)

    def desc(self, M: int, idt: int = MOE_IDX_I64) -> MoeLayerDesc:
        none = MoeWeight(None, None)
        d = MoeLayerDesc(M, self.H, self.I, self.S, self.E, self.top_k, self.BS, self.wdt, idt,
                         _weight(self.gate), _weight(self.up), _weight(self.down),
                         _weight(self.sh_gate) or none, _weight(self.sh_up) or none, _weight(self.sh_down) or none)
        d.path = self.path_request
        if self.sh_expert_gate is not None:
            g = self.sh_expert_gate
            _need(g.dtype == torch.bfloat16 and g.numel() == self.H and g.is_contiguous(),
                  "sh_expert_gate must be a contiguous bf16 vector of H elements")
            d.sh_expert_gate = g.data_ptr()
        return d

    def workspace_bytes(self, M: int, idt: int = MOE_IDX_I64) -> int:
        d = self.desc(M, idt)
        n = int(lib().moe_layer_workspace_bytes(ctypes.byref(d)))
        if n == 0:
            raise MoeError(MOE_ERR_SHAPE, lib().moe_last_error().decode())
        return n

    def workspace_layout(self, M: int, idt: int = MOE_IDX_I64):
        d = self.desc(M, idt)
        off = (ctypes.c_size_t * (MOE_LAYER_WORKSPACE_REGIONS + 1))()
        _check(lib().moe_layer_workspace_layout(ctypes.byref(d), off))
        return list(off)

    def path(self, M: int, idt: int = MOE_IDX_I64) -> int:
        """MOE_LAYER_PATH_STEPS, MOE_LAYER_PATH_SINGLE_PASS or MOE_LAYER_PATH_NARROW for M tokens."""
        d = self.desc(M, idt)
        rc = lib().moe_layer_path(ctypes.byref(d))
        if rc < 0:
            raise MoeError(rc, lib().moe_last_error().decode())
        return rc

    def alloc_workspace(self, M: int, idt: int = MOE_IDX_I64, device="cuda") -> torch.Tensor:
        return torch.empty(self.workspace_bytes(M, idt), dtype=torch.uint8, device=device)

    def workspace_views(self, ws: torch.Tensor, M: int, idt: int = MOE_IDX_I64) -> dict:
        """Typed views of the tables and of the chosen path's intermediates
        inside a used workspace (regions the path does not use are left out)."""
        off = self.workspace_layout(M, idt)
        n = M * self.top_k
        mt = moe_align_max_total(n, self.E, self.BS)
        path = self.path(M, idt)
        narrow = path == MOE_LAYER_PATH_NARROW
        sizes = {
            "sorted_token_ids": (mt,), "block_expert_ids": (mt // self.BS,), "expert_offsets": (self.E + 1,),
            "expert_counts": (self.E,), "token_to_perm": (n,), "active_experts": (moe_active_cap(n, self.E),),
            "active_count": (1,), "total": (1,),
            "act": (n if narrow else mt, self.I), "expert_out": (mt, self.H), "sh_act": (M, self.S),
            "sh_out": (M, self.H),
            "part": (-(-self.I // 64), n, self.H), "sh_part": (-(-self.S // 64), M, self.H),
        }
        used = set(TABLE_FIELDS) | {MOE_LAYER_PATH_SINGLE_PASS: {"part", "sh_part"},
                                    MOE_LAYER_PATH_NARROW: {"act", "sh_act"}}.get(
            path, {"act", "expert_out", "sh_act", "sh_out"})
        views = {}
        for i, name in enumerate(WORKSPACE_REGIONS):
            if name not in used or (name.startswith("sh_") and self.S == 0):
                continue
            shape = sizes[name]
            dt = torch.int32 if i < 8 else torch.float32
            numel = 1
            for s in shape:
                numel *= s
            views[name] = ws[off[i]:off[i] + 4 * numel].view(dt).view(*shape)
        return views

    def forward(self, x: torch.Tensor, topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
        """moe_layer_forward: align, gate+up+SiLU, down, blend on one stream, no host sync."""
        M = x.shape[0]
        _need(x.dtype == torch.bfloat16 and x.shape[1] == self.H and x.is_contiguous(), "x must be bf16 [M, H]")
        _need(topk_ids.shape == (M, self.top_k) and topk_ids.is_contiguous(), "topk_ids must be [M, top_k]")
        _need(topk_weights.shape == (M, self.top_k) and topk_weights.dtype == torch.float32
              and topk_weights.is_contiguous(), "topk_weights must be float32 [M, top_k]")
        idt = MOE_IDX_I64 if topk_ids.dtype == torch.int64 else MOE_IDX_I32
        if out is None:
            out = torch.empty(M, self.H, dtype=torch.bfloat16, device=x.device)
        if workspace is None:
            workspace = self.alloc_workspace(M, idt, x.device)
        d = self.desc(M, idt)
        _check(lib().moe_layer_forward(ctypes.byref(d), x.data_ptr(), topk_ids.data_ptr(), topk_weights.data_ptr(),
                                       out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(stream)))
        return out


def moe_layer_partials(layer: MoeLayer, x, topk_ids, workspace, stream=None) -> None:
    """First launch of the single-pass layer: tables and per-slice partial outputs into `workspace`."""
    M = x.shape[0]
    idt = MOE_IDX_I64 if topk_ids.dtype == torch.int64 else MOE_IDX_I32
    d = layer.desc(M, idt)
    _check(lib().moe_layer_partials(ctypes.byref(d), x.data_ptr(), topk_ids.data_ptr(), workspace.data_ptr(),
                                    workspace.numel(), _stream(stream)))


def moe_layer_blend_partials(layer: MoeLayer, topk_ids, topk_weights, out, workspace, stream=None, x=None):
    """Second launch of the single-pass layer: sum the partials, blend into `out`
    (x is needed when the layer has a shared gate vector)."""
    M = topk_ids.shape[0]
    idt = MOE_IDX_I64 if topk_ids.dtype == torch.int64 else MOE_IDX_I32
    d = layer.desc(M, idt)
    _check(lib().moe_layer_blend_partials(ctypes.byref(d), None if x is None else x.data_ptr(), topk_ids.data_ptr(),
                                          topk_weights.data_ptr(), out.data_ptr(), workspace.data_ptr(),
                                          workspace.numel(), _stream(stream)))
    return out


def moe_router_topk(x, router_w, top_k: int, ids_dtype=torch.int64, logits=None, stream=None):
    """Per-row router: float32 logits of bf16 x [M, H] against the bf16 gate
    weight [E, H], each row's top_k experts (larger logit first, ties to the
    lower expert) and their softmax weights over the chosen logits.  Returns
    (topk_ids [M, top_k] of ids_dtype, topk_weights float32 [M, top_k],
    logits float32 [M, E])."""
    M, H = x.shape
    E = router_w.shape[0]
    if router_w.shape[1] != H or x.dtype != torch.bfloat16 or router_w.dtype != torch.bfloat16:
        raise ValueError("x [M, H] and router_w [E, H] must both be bfloat16 with the same H")
    if not (x.is_contiguous() and router_w.is_contiguous()):
        raise ValueError("x and router_w must be contiguous")
    dev = x.device
    if logits is None:
        logits = torch.empty(M, E, dtype=torch.float32, device=dev)
    ids = torch.empty(M, top_k, dtype=ids_dtype, device=dev)
    wts = torch.empty(M, top_k, dtype=torch.float32, device=dev)
    idt = MOE_IDX_I64 if ids_dtype == torch.int64 else MOE_IDX_I32
    _check(lib().moe_router_topk(x.data_ptr(), router_w.data_ptr(), M, H, E, top_k, logits.data_ptr(), ids.data_ptr(),
                                 idt, wts.data_ptr(), _stream(stream)))
    return ids, wts, logits


def moe_stream_read_probe(src, sink, blocks: int = 2048, stream=None):
    """One plain streaming read of the whole of `src` (a contiguous device
    tensor, size a multiple of 16 bytes); `sink` is an int32 device tensor of at
    least 4 * blocks elements.  A measurement aid: the read rate it reaches is
    the ceiling the layer's weight stream is compared with."""
    if sink.numel() < 4 * blocks:
        raise ValueError("sink needs at least 4 * blocks int32 elements")
    _check(lib().moe_stream_read_probe(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(), blocks,
                                       _stream(stream)))


def moe_layer_workspace_bytes(layer: MoeLayer, M: int, idt: int = MOE_IDX_I64) -> int:
    return layer.workspace_bytes(M, idt)


def moe_layer_forward(layer: MoeLayer, x, topk_ids, topk_weights, out=None, workspace=None, stream=None):
    return layer.forward(x, topk_ids, topk_weights, out, workspace, stream)
