"""Stage a synthetic layer in GPU memory (torch tensors), expert by expert.

Only the experts that received at least one slot are generated; every other
expert is filled with NaN (bf16/fp32 NaN, e4m3 code 0x7F, NaN scales; FP4 codes have
no NaN, so there the UE8M0 scales 0xFF carry it), so a kernel that touched an
unselected expert would poison its output.  This also
keeps host memory and generation time proportional to the active experts.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from .layers import Spec, active_experts, expert_down, expert_gate_up, hidden, routing

_TORCH_W = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8, "fp4": torch.uint8}


def host_to_tensor(a: np.ndarray, fmt: str) -> torch.Tensor:
    """Host array in a storage format -> CPU tensor of the matching torch dtype."""
    if fmt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a))


def _poison(t: torch.Tensor, fmt: str):
    if fmt == "fp8":
        t.fill_(0x7F)
    elif fmt == "fp4":
        t.fill_(0x77)          # (6, 6); the NaN comes from the scales
    elif fmt == "ue8m0":
        t.fill_(0xFF)
    else:
        t.fill_(float("nan"))


def device_layer(spec: Spec, device="cuda", threads: int = 16, poison_inactive: bool = True) -> dict:
    """All inputs of `spec` as device tensors.

    Keys: spec, x, idx, w, w_gate_up, w_down, (w_gate_up_scale, w_down_scale),
    idx_host, w_host, x_host, active (sorted active expert ids).
    """
    device = torch.device(device)
    idx, w = routing(spec)
    x = hidden(spec)
    active = active_experts(idx, spec.E)
    wdt = _TORCH_W[spec.weight]
    out = {"spec": spec, "idx_host": idx, "w_host": w, "x_host": x, "active": active}
    out["x"] = host_to_tensor(x, spec.act).to(device)
    out["idx"] = torch.from_numpy(idx).to(device)
    out["w"] = torch.from_numpy(w).to(device)
    E, H, I = spec.E, spec.H, spec.I
    fp4 = spec.weight == "fp4"
    gu = torch.empty((E, 2 * I, H // 2 if fp4 else H), dtype=wdt, device=device)
    dn = torch.empty((E, H, I // 2 if fp4 else I), dtype=wdt, device=device)
    fp8 = spec.weight in ("fp8", "fp4")     # (weights with scale tensors)
    if fp4:
        gus = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=device)
        dns = torch.empty((E, H, I // 32), dtype=torch.uint8, device=device)
    elif fp8:
        sdt = torch.float32 if spec.scale == "f32" else torch.uint8
        gus = torch.empty((E, 2 * I // 128, H // 128), dtype=sdt, device=device)
        dns = torch.empty((E, H // 128, I // 128), dtype=sdt, device=device)
    todo = list(active) if poison_inactive else list(range(E))
    if poison_inactive:
        mask = np.ones(E, dtype=bool)
        mask[active] = False
        for e in np.nonzero(mask)[0]:
            _poison(gu[e], spec.weight)
            _poison(dn[e], spec.weight)
            if fp8:
                _poison(gus[e], spec.scale)
                _poison(dns[e], spec.scale)

    def make(e):
        return e, expert_gate_up(spec, e), expert_down(spec, e)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        for i in range(0, len(todo), threads):
            for e, g, d in ex.map(make, todo[i:i + threads]):
                if fp8:
                    gu[e].copy_(torch.from_numpy(g[0]))
                    gus[e].copy_(torch.from_numpy(g[1]))
                    dn[e].copy_(torch.from_numpy(d[0]))
                    dns[e].copy_(torch.from_numpy(d[1]))
                else:
                    gu[e].copy_(host_to_tensor(g, spec.weight))
                    dn[e].copy_(host_to_tensor(d, spec.weight))
    out["w_gate_up"], out["w_down"] = gu, dn
    if fp8:
        out["w_gate_up_scale"], out["w_down_scale"] = gus, dns
    if device.type == "cuda":
        torch.cuda.synchronize(device)
    return out
