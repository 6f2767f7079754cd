"""Key-coverage checks: exact closed-form outputs that see every key.

With K = 0 every score is 0, so every visible key gets the same softmax
weight and attention returns the plain mean of V over the visible keys
("28. Grouped-Query Attention (GQA)", *Step-by-Step Approach*: the softmax
runs over every key the mask leaves visible; the oracle pin
pin_zero_keys_give_mean fixes this closed form, and test_coverage_cpu ties
the functions here to the oracle).

V holds the integer pattern of workloads.key_pattern_rows, so the mean is a
quotient of two integers below 2^24.  The kernels reach it exactly: every
weight is 2^0 = 1, every product and partial sum of integers below 2^24 is
exact in fp32 whatever the order (including the merge of key splits, whose
rescale factors are all 2^0), and the final division is correctly rounded.
So the fp32 output must equal the fp32 rounding of the exact quotient bit for
bit, and a 16-bit output the 16-bit rounding of that fp32 value.

The expected quotient is computed here as an fp64 division of exact int64
sums, then rounded to fp32.  That double rounding is safe: a quotient a/c
with c <= 2^17 keys that is not an fp32 rounding midpoint lies at least
2^-25/c >= 2^-42 (relative) from every midpoint, far more than the 2^-53
relative error of the fp64 division, and an exact midpoint is representable
in fp64.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle


def band_ranges(N, M, q_offset=0, window_left=-1, window_right=-1):
    """(lo, hi) int64 [N]: keys lo[i] <= j < hi[i] are visible to query i
    under the band rule of the banded prefill (a negative window leaves that
    side open), clamped to [0, M].  Causal is (0, -1, 0); no band is
    (0, -1, -1)."""
    pos = np.arange(N, dtype=np.int64) + q_offset
    lo = np.zeros(N, dtype=np.int64) if window_left < 0 else np.clip(pos - window_left, 0, M)
    hi = np.full(N, M, dtype=np.int64) if window_right < 0 else np.clip(pos + window_right + 1, 0, M)
    return lo, np.maximum(hi, lo)


def exact_means(v, H, lo, hi):
    """fp32 [B, H, N, D]: mean of v[b, h // g, lo[b, i]:hi[b, i], :] per query
    row, correctly rounded from the exact quotient; NaN where no key is
    visible.  v: integer-valued tensor or ndarray [B, H_kv, M, D]; lo, hi:
    int arrays [B, N]."""
    B, H_kv, M, D = v.shape
    g = H // H_kv
    N = lo.shape[1]
    out = np.empty((B, H, N, D), dtype=np.float32)
    for b in range(B):
        vb = v[b]
        if isinstance(vb, torch.Tensor):
            vb = vb.float().numpy()
        vb = np.asarray(vb).astype(np.int64)                  # exact: small integers
        pre = np.zeros((H_kv, M + 1, D), dtype=np.int64)
        np.cumsum(vb, axis=1, out=pre[:, 1:, :])
        s = pre[:, hi[b], :] - pre[:, lo[b], :]                # [H_kv, N, D]
        cnt = (hi[b] - lo[b]).astype(np.float64)[None, :, None]
        with np.errstate(invalid="ignore", divide="ignore"):
            mean = np.where(cnt > 0, s.astype(np.float64) / cnt, np.nan)
        out[b] = np.repeat(mean, g, axis=0).astype(np.float32)
    return out


def paged_exact_means(q_shape, k_pool, v_pool, block_table, kv_len):
    """Expected decode output of a paged key-coverage check: the pool is
    gathered per sequence by the oracle's gather_paged, then exact_means over
    keys [0, kv_len[b])."""
    B, H, _, _ = q_shape
    _, v, _ = oracle.gather_paged(k_pool.float().numpy(), v_pool.float().numpy(),
                                  block_table.numpy(), kv_len.numpy())
    M = v.shape[2]
    lens = np.clip(kv_len.numpy().astype(np.int64), 0, M)
    lo = np.zeros((B, 1), dtype=np.int64)
    hi = lens[:, None]
    return exact_means(v, H, lo, hi)


def mismatches(got, want_f32):
    """Number of elements where the GPU output differs from the exact
    expectation (want rounded to got's dtype first), NaN matching NaN, plus a
    description of the first few."""
    want_t = torch.from_numpy(want_f32)
    if got.dtype != torch.float32:
        want_t = want_t.to(got.dtype)
    g = got.detach().cpu().float().numpy()
    w = want_t.float().numpy()
    bad = ~((g == w) | (np.isnan(g) & np.isnan(w)))
    n = int(bad.sum())
    if n == 0:
        return 0, ""
    idx = np.argwhere(bad)[:5]
    desc = "; ".join(f"{tuple(int(x) for x in i)}: got {g[tuple(i)]!r} want {w[tuple(i)]!r}"
                     for i in idx)
    return n, desc


def assert_exact(got, want_f32, what):
    n, desc = mismatches(got, want_f32)
    assert n == 0, f"{what}: {n} elements differ from the exact visible-key mean ({desc})"
