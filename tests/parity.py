"""Shared helpers for the GPU parity tests: run the HIP path and the fp64
oracle on the same seeded inputs and compare element by element."""

from __future__ import annotations

import numpy as np
import torch

import oracle

# Tolerances (max abs error against the fp64 oracle run on the same,
# already-rounded inputs): fp32 inputs 1e-4; bf16 inputs with fp32
# accumulation 2e-2; fp16 inputs 5e-3 (rounding the weights to fp16 costs at
# most 2^-11 max|v|, about 2.4e-3 for N(0,1) values, and rounding an output
# below 4 in magnitude at most 2^-9 = 2e-3).
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2, torch.float16: 5e-3}


def np64(t):
    if t is None:
        return None
    if t.dtype == torch.bool:
        return t.cpu().numpy()
    return t.detach().float().cpu().numpy().astype(np.float64)


def to_dev(*ts):
    return [None if t is None else t.cuda() for t in ts]


def compare(got, ref, tol, what=""):
    """got: torch tensor (any device), ref: float64 ndarray.  NaN must match
    NaN exactly (rows with no visible key); finite entries within tol."""
    g = got.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(g), nan_ref), f"{what}: NaN pattern differs"
    fin = ~nan_ref
    if not fin.any():
        return 0.0, 0.0
    err = np.abs(g[fin] - ref[fin])
    mx = float(err.max())
    rel_rms = float(np.sqrt((err ** 2).sum() / max((ref[fin] ** 2).sum(), 1e-300)))
    assert mx <= tol, f"{what}: max abs err {mx:.3e} > {tol:.1e} (rel rms {rel_rms:.2e})"
    return mx, rel_rms


def oracle_out(q, k, v, mask=None, causal=False):
    return oracle.gqa(np64(q), np64(k), np64(v), np64(mask), causal)
