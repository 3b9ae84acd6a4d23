"""Moving bf16 bit arrays between numpy and the GPU, and running the library
(through the C-ABI binding) on a workload. Test infrastructure only."""
from __future__ import annotations

import numpy as np
import torch

import invariant_rmsnorm_amd as irn


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev_f32(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def run_fwd_bwd(p, gres: bool = False):
    """GPU forward (plain) and backward on a synth Problem; host results."""
    x, gamma = dev_bf16(p.x), dev_f32(p.gamma)
    y, rstd = irn.rmsnorm_fwd(x, gamma, p.zero_centered, p.eps)
    out = {"y": host_bits(y), "rstd": rstd.cpu().numpy()}
    if p.g is not None:
        g = dev_bf16(p.g)
        gr = dev_bf16(p.gres) if (gres and p.gres is not None) else None
        dx, dg = irn.rmsnorm_bwd(g, x, rstd, gamma, p.zero_centered, g_residual=gr)
        out["dx"], out["dgamma"] = host_bits(dx), dg.cpu().numpy()
    torch.cuda.synchronize()
    return out
