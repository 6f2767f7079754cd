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

# Bound on the relative RMS error ||got - ref||_2 / ||ref||_2, per input type.
# A max-abs bar alone is loose where the outputs are small (a decode over
# 32768 keys has outputs of std 0.009), so a kernel that skipped a range of
# keys could pass it.  With 16-bit inputs two roundings to the input type
# reach the output: the softmax weights before the P.V product and the
# output itself.  RNE rounding of a value x in [2^e, 2^(e+1)) has an absolute
# error uniform on +-ulp/2 with ulp = 2^(e-p+1) (p = 8 bits for bf16, 11 for
# fp16), so its relative RMS error is ulp/sqrt(12) * E[1/x^2]^(1/2) =
# 2^(1-p)/sqrt(12)/sqrt(2) for x uniform in the binade: 1.6e-3 for bf16,
# 2.0e-4 for fp16.  The weight rounding enters the output as
# sum_j w_j eps_j v_j, whose RMS relative to o = sum_j w_j v_j is the same
# figure for independent v_j, so the two together give sqrt(2) times it:
# 2.3e-3 (bf16) and 2.8e-4 (fp16).  The bounds leave a factor 3.5 (bf16) and
# 5 (fp16) above that.  fp32 inputs keep everything in fp32 (rounding error
# ~1e-7 per operation); 1e-5 leaves room for accumulation over long key
# ranges.  Skipping keys moves the output by far more: dropping 1/8 of the
# keys of a 32768-key decode gives a relative RMS change of about 0.35, one
# 128-key round per key split about 0.09.
REL_RMS = {torch.float32: 1e-5, torch.bfloat16: 8e-3, torch.float16: 1.5e-3}
_REL_RMS_BY_TOL = {TOL[t]: REL_RMS[t] for t in TOL}

# Every comparison made in this process: (what, dtype of got, max abs err,
# relative RMS error), written out by the test session when asked to.
STATS = []


def np64(t):
    if t is None:
        return None
    if t.dtype == torch.bool:
        return t.cpu().numpy()
    return t.detach().float().cpu().numpy().astype(np.float64)


def to_dev(*ts):
    return [None if t is None else t.cuda() for t in ts]


def rel_rms_error(got, ref):
    """||got - ref||_2 / ||ref||_2 over the finite entries of ref (float64
    ndarrays of the same shape)."""
    fin = ~np.isnan(ref)
    err = got[fin] - ref[fin]
    return float(np.sqrt((err ** 2).sum() / max((ref[fin] ** 2).sum(), 1e-300)))


def compare(got, ref, tol, what="", rel_rms=None):
    """got: torch tensor (any device), ref: float64 ndarray.  NaN must match
    NaN exactly (rows with no visible key); finite entries within tol of the
    reference, and the relative RMS error within rel_rms (by default the
    bound of the input type whose max-abs tolerance is tol)."""
    g = got.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(g), nan_ref), f"{what}: NaN pattern differs"
    fin = ~nan_ref
    if not fin.any():
        return 0.0, 0.0
    err = np.abs(g[fin] - ref[fin])
    mx = float(err.max())
    rr = rel_rms_error(g, ref)
    STATS.append((what, str(got.dtype), tol, mx, rr))
    assert mx <= tol, f"{what}: max abs err {mx:.3e} > {tol:.1e} (rel rms {rr:.2e})"
    bound = rel_rms if rel_rms is not None else _REL_RMS_BY_TOL.get(tol)
    if bound is not None:
        assert rr <= bound, f"{what}: relative RMS error {rr:.3e} > {bound:.1e} (max abs {mx:.2e})"
    return mx, rr


def oracle_out(q, k, v, mask=None, causal=False):
    return oracle.gqa(np64(q), np64(k), np64(v), np64(mask), causal)
