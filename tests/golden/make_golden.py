"""Writes oracle_tiny_sha256.json: SHA-256 digests of the CPU oracle's
outputs on the small seeded fixtures (T=16, D=128; both weight conventions;
residual, gated, residual-gradient and fused add-norm forms; and rows whose
length is not a multiple of 8, D = 13 and 100), plus digests of the inputs.

It calls only the oracle and the input generator. A later change that moves
any of these bytes must be explained in the commit that regenerates the file.
Run from the repository root:  python tests/golden/make_golden.py
"""
from __future__ import annotations

import hashlib
import json
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[2]
sys.path.insert(0, str(ROOT))

import oracle  # noqa: E402
from synth import workloads as wl  # noqa: E402

OUT = Path(__file__).resolve().parent / "oracle_tiny_sha256.json"


def digest(a) -> str:
    return hashlib.sha256(memoryview(a).cast("B")).hexdigest()


def manifest() -> dict:
    m = {}
    cases = [(zc, 128, 1001) for zc in (False, True)] + [(False, 13, 1013), (True, 100, 1100)]
    for zc, D, seed in cases:
        p = wl.tiny(zc, D=D, seed=seed, with_gres=True, with_gate=True, with_residual=True)
        key = p.name
        y, r = oracle.fwd(p.x, p.gamma, zc, p.eps)
        _, res, _ = oracle.residual_fwd(p.x, p.gamma, zc, p.eps)
        out, _ = oracle.gated_fwd(p.x, p.z, p.gamma, zc, p.eps)
        dx, dg = oracle.bwd(p.g, p.x, r, p.gamma, zc)
        dxr = oracle.bwd_dx(p.g, p.x, r, p.gamma, zc, p.gres)
        ay, arout, ar = oracle.add_fwd(p.x, p.residual, p.gamma, zc, p.eps)
        adh, adg = oracle.add_bwd(p.g, p.x, p.residual, ar, p.gamma, zc, g_rout=p.gres)
        m[key] = {
            "inputs": {n: digest(a) for n, a in
                       (("x", p.x), ("g", p.g), ("gres", p.gres), ("z", p.z),
                        ("gamma", p.gamma), ("residual", p.residual))},
            "y": digest(y), "rstd": digest(r), "residual_out": digest(res),
            "gated_out": digest(out), "dx": digest(dx), "dgamma": digest(dg),
            "dx_with_gres": digest(dxr),
            "add_y": digest(ay), "add_residual_out": digest(arout), "add_rstd": digest(ar),
            "add_dh": digest(adh), "add_dgamma": digest(adg),
        }
    return m


if __name__ == "__main__":
    OUT.write_text(json.dumps(manifest(), indent=1, sort_keys=True) + "\n")
    print("wrote", OUT)
