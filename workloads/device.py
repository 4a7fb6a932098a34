"""Device copies of the seeded workloads (torch tensors on a GPU).

Plumbing only: the generators of ``gen.py`` draw the values, this module
places them in device memory in the layouts the library takes
(``[E, N, K]`` weights, ``[E, N/128, K/128]`` scales, bf16 activations,
int64 ids, float32 router weights).
"""

from __future__ import annotations

import threading

import numpy as np

from .gen import MoeConfig, fill_expert_weights, routing, shared_matrix, weight_shape, x_bf16


def _torch():
    import torch

    return torch


class DeviceWeights:
    """Every expert's gate/up/down (and the shared expert's) on ``device``.
    With ``keep_host`` the raw generated arrays are kept too, keyed
    ``(which, e)``, so a checker can use the very same values."""

    def __init__(self, cfg: MoeConfig, device="cuda", keep_host: bool = False, threads: int = 8):
        torch = _torch()
        self.cfg = cfg
        fp8 = cfg.wdt in ("fp8", "fp8_rows", "mxfp4")  # byte-coded weights with scales
        rows = cfg.wdt == "fp8_rows"  # one scale per row [E, N] instead of per 128x128 block
        mx = cfg.wdt == "mxfp4"       # packed 4-bit codes [E, N, K/2], E8M0 bytes [E, N, K/32]
        wdt = torch.uint8 if fp8 else torch.bfloat16
        self.host = {} if keep_host else None
        lock = threading.Lock()
        self.w, self.s = {}, {}
        for which in ("gate", "up", "down"):
            N, K = weight_shape(cfg, which)
            self.w[which] = torch.empty(cfg.E, N, K // 2 if mx else K, dtype=wdt, device=device)
            sshape = (cfg.E, N) if rows else ((cfg.E, N, K // 32) if mx else (cfg.E, N // 128, K // 128))
            sdt = torch.uint8 if mx else torch.float32
            self.s[which] = torch.empty(*sshape, dtype=sdt, device=device) if fp8 else None

            def sink(e, bits, sc, which=which):
                src = torch.from_numpy(bits) if fp8 else torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
                self.w[which][e].copy_(src)
                if fp8:
                    self.s[which][e].copy_(torch.from_numpy(sc))
                if self.host is not None:
                    with lock:
                        self.host[(which, e)] = (bits, sc)

            fill_expert_weights(cfg, which, sink, threads=threads)
        self.sh = {}
        self.sh_host = {}
        if cfg.S:
            for which in ("gate", "up", "down"):
                bits, sc = shared_matrix(cfg, which)
                self.sh_host[which] = (bits, sc)
                src = torch.from_numpy(bits) if fp8 else torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
                self.sh[which] = (src.to(device), torch.from_numpy(sc).to(device) if fp8 else None)
        if str(device).startswith("cuda"):
            torch.cuda.synchronize()

    def weight(self, which):
        return (self.w[which], self.s[which])

    def clone(self) -> "DeviceWeights":
        """A second copy of the same weights at other device addresses."""
        other = object.__new__(DeviceWeights)
        other.cfg = self.cfg
        other.host = None
        other.sh_host = {}
        other.w = {k: v.clone() for k, v in self.w.items()}
        other.s = {k: (None if v is None else v.clone()) for k, v in self.s.items()}
        other.sh = {k: (w.clone(), None if s is None else s.clone()) for k, (w, s) in self.sh.items()}
        return other

    def algorithmic_bytes(self, ids: np.ndarray, M: int = None) -> dict:
        """Weight bytes one layer call must stream for routing ``ids``: every
        active expert's three matrices (and their scales) once, plus the shared
        expert's."""
        cfg = self.cfg
        E = cfg.E
        flat = np.asarray(ids).reshape(-1)
        active = int(np.unique(flat[(flat >= 0) & (flat < E)]).size)
        esz = {"fp8": 1.0, "fp8_rows": 1.0, "mxfp4": 0.5}.get(cfg.wdt, 2.0)

        def mat(N, K):
            b = int(N * K * esz)
            if cfg.wdt == "fp8":
                b += (N // 128) * (K // 128) * 4
            elif cfg.wdt == "fp8_rows":
                b += N * 4
            elif cfg.wdt == "mxfp4":
                b += N * (K // 32)
            return b

        gate_up = 2 * mat(cfg.I, cfg.H) * active
        down = mat(cfg.H, cfg.I) * active
        if cfg.S:
            gate_up += 2 * mat(cfg.S, cfg.H)
            down += mat(cfg.H, cfg.S)
        return {"active": active, "gate_up": gate_up, "down": down, "total": gate_up + down}


def device_inputs(cfg: MoeConfig, device="cuda"):
    """(host arrays, device tensors) of x, topk_ids (int64) and topk_weights."""
    torch = _torch()
    x = x_bf16(cfg)
    ids, w = routing(cfg)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(device)
    it = torch.from_numpy(ids).to(device)
    wt = torch.from_numpy(w).to(device)
    return (x, ids, w), (xt, it, wt)
