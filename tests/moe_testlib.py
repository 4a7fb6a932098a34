"""Helpers shared by the GPU tests: device copies of the seeded workloads,
oracle adapters and the parity tolerance.

Inputs come only from ``workloads`` (the seeded generators); expected values
come only from ``oracle``.  Nothing here computes any part of the path.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads
from workloads import MoeConfig
from workloads.device import DeviceWeights, device_inputs  # noqa: F401


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def tolerance_ok(got: np.ndarray, ref: np.ndarray):
    """The parity bar for floating point: max|gpu - oracle| <= 2e-2 * rms(oracle) + 1e-3."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    bound = 2e-2 * rms + 1e-3
    return err <= bound, err, bound


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().float().numpy().astype(np.float64)


class DeviceModel(DeviceWeights):
    """One config's expert weights on the GPU plus oracle adapters that return
    the very same generated arrays (kept on the host for small configs,
    regenerated per expert for large ones)."""

    def __init__(self, cfg: MoeConfig, device="cuda", keep_host: bool = True, threads: int = 8):
        super().__init__(cfg, device=device, keep_host=keep_host, threads=threads)

    def layer(self, sh_expert_gate=None):
        from mixture_experts_routing_align_amd import MoeLayer

        sh = self.sh or {}
        return MoeLayer(self.weight("gate"), self.weight("up"), self.weight("down"), self.cfg.top_k, self.cfg.BS,
                        sh.get("gate"), sh.get("up"), sh.get("down"), sh_expert_gate=sh_expert_gate)

    def tiled_layer(self):
        """The layer with tiled weights (built once per model)."""
        if getattr(self, "_tiled", None) is None:
            self._tiled = self.layer().tiled()
        return self._tiled

    def routed_weight(self, which, e):
        """The generated (bits, scales) of expert e's matrix `which`: kept on the
        host for small configs; for large ones read back from the row-major
        device copy, which holds exactly the generator's bits (torch copied
        them there; no kernel of the library wrote them)."""
        if self.host is not None:
            return self.host[(which, e)]
        w, s = self.weight(which)
        bits = w[e].cpu().numpy()
        if w.dtype == torch.bfloat16:
            bits = w[e].view(torch.int16).cpu().numpy().view(np.uint16)
        return bits, (None if s is None else s[e].cpu().numpy())

    def shared_weight(self):
        if not self.cfg.S:
            return None
        return lambda which: self.sh_host[which]


def oracle_layer(model: DeviceModel, x, ids, w, tokens=None, sh_gate_bits=None):
    cfg = model.cfg
    return oracle.moe_layer(x, ids, w, cfg.E, cfg.BS, cfg.wdt, model.routed_weight, model.shared_weight(),
                            tokens=tokens, sh_gate_bits=sh_gate_bits)


TABLE_KEYS = ("sorted_token_ids", "block_expert_ids", "expert_offsets", "expert_counts", "token_to_perm",
              "active_experts")


def compare_tables(gpu_tables: dict, ref: dict) -> None:
    """Bit-exact comparison of every alignment table (gpu_tables: name -> tensor)."""
    for key in TABLE_KEYS:
        g = gpu_tables[key].cpu().numpy().astype(np.int64)
        r = np.asarray(ref[key], dtype=np.int64)
        assert g.shape == r.shape, (key, g.shape, r.shape)
        if not np.array_equal(g, r):
            bad = np.flatnonzero(g != r)
            raise AssertionError(f"{key}: {bad.size} entries differ, first at {bad[:5]}: gpu {g[bad[:5]]} "
                                 f"oracle {r[bad[:5]]}")
    assert int(gpu_tables["active_count"].item()) == int(ref["active_count"])
    assert int(gpu_tables["total"].item()) == int(ref["total"])


def separate_steps(moe, layer, xt, it, wt):
    """align, gate+up, down and blend called one by one through their entry points."""
    M = xt.shape[0]
    t = moe.moe_align(it, layer.E, layer.BS)
    mt = t.sorted_token_ids.numel()
    act = torch.empty(mt, layer.I, device="cuda")
    eo = torch.empty(mt, layer.H, device="cuda")
    sh_act = sh_out = None
    if layer.S:
        sh_act = torch.empty(M, layer.S, device="cuda")
        sh_out = torch.empty(M, layer.H, device="cuda")
    moe.moe_grouped_gate_up_silu(xt, layer.gate, layer.up, t, act, layer.top_k, layer.BS, layer.sh_gate, layer.sh_up,
                                 sh_act)
    moe.moe_grouped_down(act, layer.down, t, eo, M, layer.top_k, layer.BS, layer.sh_down, sh_act, sh_out)
    out = torch.empty(M, layer.H, dtype=torch.bfloat16, device="cuda")
    moe.moe_blend(out, eo, wt, t.token_to_perm, sh_out)
    torch.cuda.synchronize()
    return out, t
