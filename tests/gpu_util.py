"""Helpers shared by the GPU tests: host->device marshalling and the tolerances.

Tolerances (bf16 inputs, fp32 accumulation):
* contract: max |out - ref| <= 1e-2 and max |lse - ref| <= 1e-3;
* stricter, because the contract is loose next to the outputs' scale (outputs
  of the N(0,1)/sqrt(128) workloads are ~1e-3): max |out - ref| <= 1e-2 *
  max |ref|. Each probability is rounded to bf16 before the PV product
  (relative 2^-9) and the output is rounded to bf16 (2^-9 of its magnitude),
  so 1e-2 of the largest output leaves a ~5x margin.
* lse: fp32 sums over up to 1e5 terms, split and merged: ~1e-6 relative of
  ~11.5; gate at 5e-5 absolute.
* fp32 inputs: products and sums in fp32; gate at 2e-5 of max |ref| and 2e-5
  on lse.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None

CONTRACT_OUT = 1e-2
CONTRACT_LSE = 1e-3
TOL = {
    "bf16": dict(out_rel=1e-2, lse=5e-5),
    "f32": dict(out_rel=2e-5, lse=2e-5),
}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    if a.dtype == np.int32:
        return torch.from_numpy(a).to(DEV)
    return torch.from_numpy(a.astype(np.float32)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def check_attn(out, lse, ref_out, ref_lse, dtype: str, label: str):
    got = to_host(out)
    gl = to_host(lse)
    assert np.isfinite(got).all() and np.isfinite(gl).all(), f"{label}: non-finite output"
    err = np.abs(got - ref_out).max()
    lerr = np.abs(gl - ref_lse).max()
    scale = np.abs(ref_out).max()
    say(f"  {label}: max|dout| {err:.3e} (max|ref| {scale:.3e}, rel {err / scale:.3e}); max|dlse| {lerr:.3e}")
    assert err <= CONTRACT_OUT, f"{label}: out error {err} > contract {CONTRACT_OUT}"
    assert lerr <= CONTRACT_LSE, f"{label}: lse error {lerr} > contract {CONTRACT_LSE}"
    t = TOL[dtype]
    assert err <= t["out_rel"] * scale, f"{label}: out error {err} > {t['out_rel']} * max|ref|"
    assert lerr <= t["lse"], f"{label}: lse error {lerr} > {t['lse']}"
    return err, lerr
