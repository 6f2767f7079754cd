"""CPU checks of the key-coverage closed forms (tests/coverage.py) and of the
parity bars: the closed forms equal the fp64 oracle, and outputs of a
kernel that skipped, repeated or shifted keys fail both the exact
key-coverage check and the relative-RMS bound of compare()."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import coverage
from tests.parity import REL_RMS, rel_rms_error


def _oracle_k0(q, k, v, mask=None, causal=False):
    f = lambda t: t.float().numpy().astype(np.float64)   # noqa: E731
    return oracle.gqa(f(q), f(k), f(v), None if mask is None else mask.numpy(), causal)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_exact_means_equal_oracle_decode(dtype):
    B, H, H_kv, M, D = 3, 8, 2, 700, 16
    q, k, v = workloads.key_coverage_inputs(B, H, H_kv, 1, M, D, dtype)
    lo = np.zeros((B, 1), dtype=np.int64)
    hi = np.full((B, 1), M, dtype=np.int64)
    want = coverage.exact_means(v, H, lo, hi)
    np.testing.assert_allclose(want, _oracle_k0(q, k, v), rtol=1e-6, atol=0)


@pytest.mark.parametrize("band", [(0, -1, 0), (0, 9, 0), (30, -1, 0), (-5, 3, 4), (0, -1, -1)])
def test_exact_means_equal_oracle_band(band):
    B, H, H_kv, N, M, D = 2, 6, 3, 40, 70, 8
    q, k, v = workloads.key_coverage_inputs(B, H, H_kv, N, M, D, torch.bfloat16)
    lo, hi = coverage.band_ranges(N, M, *band)
    want = coverage.exact_means(v, H, np.tile(lo, (B, 1)), np.tile(hi, (B, 1)))
    f = lambda t: t.float().numpy().astype(np.float64)   # noqa: E731
    ref = oracle.gqa_band(f(q), f(k), f(v), None, *band)
    assert np.array_equal(np.isnan(want), np.isnan(ref))
    fin = ~np.isnan(ref)
    np.testing.assert_allclose(want[fin], ref[fin], rtol=1e-6, atol=0)


def test_paged_exact_means_equal_oracle():
    w = workloads.PagedWorkload("cov_small", 61, 5, 8, 2, 100, 16, 16, "bf16")
    q, kp, vp, table, lens = workloads.key_coverage_paged(w)
    want = coverage.paged_exact_means(q.shape, kp, vp, table, lens)
    f = lambda t: t.float().numpy().astype(np.float64)   # noqa: E731
    ref = oracle.gqa_paged(f(q), f(kp), f(vp), table.numpy(), lens.numpy())
    np.testing.assert_allclose(want, ref, rtol=1e-6, atol=0)


def test_pattern_has_no_power_of_two_period():
    """Dropping an aligned range of 2^k keys must change the mean: the
    pattern's period in the key index is the prime 251."""
    r = workloads.key_pattern_rows(0, 1, 0, 4096, 4)[0].numpy()
    for span in (16, 32, 64, 128, 256, 512, 1024, 2048):
        assert not np.array_equal(r[:span], r[span:2 * span]), span


def _kernel_like(v, H, key_sets):
    """Output of a kernel that averaged V over key_sets[b] (a list of key
    indices, repeats allowed) for every head: fp32 of the exact mean."""
    B, H_kv, M, D = v.shape
    g = H // H_kv
    out = np.empty((B, H, 1, D), dtype=np.float32)
    for b in range(B):
        vb = v[b].float().numpy().astype(np.int64)[:, key_sets[b], :]   # [H_kv, n, D]
        mean = vb.sum(axis=1) / float(len(key_sets[b]))
        out[b, :, 0, :] = np.repeat(mean, g, axis=0).astype(np.float32)
    return torch.from_numpy(out)


# (M, key splits, keys per split) of the benchmarked decode plans: the
# Mistral-7B shape splits 4096 keys in two, the Llama-2-70B shape 32768 keys
# in two; a workgroup walks its split in rounds of 128 keys.
@pytest.mark.parametrize("M,splits", [(4096, 2), (32768, 2), (65536, 64)])
def test_key_coverage_check_catches_skipped_keys(M, splits):
    B, H, H_kv, D = 2, 4, 2, 128
    q, k, v = workloads.key_coverage_inputs(B, H, H_kv, 1, M, D, torch.bfloat16)
    lo = np.zeros((B, 1), dtype=np.int64)
    hi = np.full((B, 1), M, dtype=np.int64)
    want = coverage.exact_means(v, H, lo, hi)
    all_keys = list(range(M))
    kps = M // splits
    assert coverage.mismatches(_kernel_like(v, H, [all_keys] * B), want)[0] == 0
    mutants = {
        "one 128-key round per split dropped":
            [j for j in all_keys if j % kps < kps - 128],
        "first round of each split dropped":
            [j for j in all_keys if j % kps >= 128],
        "last eighth dropped": all_keys[: M - M // 8],
        "first key dropped": all_keys[1:],
        "last key dropped": all_keys[:-1],
        "a round read twice": all_keys + list(range(128)),
        "range shifted by one (last key read twice)": all_keys[1:] + [M - 1],
    }
    size = B * H * D
    for name, keys in mutants.items():
        n, _ = coverage.mismatches(_kernel_like(v, H, [keys] * B), want)
        assert n >= size // 2, f"{name}: only {n} of {size} outputs differ"


def test_rel_rms_bound_catches_skipped_keys():
    """With random inputs at the Llama-2-70B decode length (M = 32768), a
    decode that skipped one 128-key round per key split, or the last eighth
    of the keys, moves the output far beyond the relative-RMS bound of bf16
    inputs, although its max abs error stays under the 2e-2 bar."""
    B, H, H_kv, M, D = 1, 8, 1, 32768, 128
    q, k, v, _ = workloads.random_case(5, B, H, H_kv, 1, M, D, torch.bfloat16)
    f = lambda t: t.float().numpy().astype(np.float64)   # noqa: E731
    qn, kn, vn = f(q), f(k), f(v)
    ref = oracle.gqa(qn, kn, vn)
    kps = M // 2
    for name, keep in {
        "one round per split": np.array([j % kps < kps - 128 for j in range(M)]),
        "last eighth": np.arange(M) < M - M // 8,
    }.items():
        bad = oracle.gqa(qn, kn, vn, np.broadcast_to(keep, (B, 1, M)).copy())
        rr = rel_rms_error(bad, ref)
        assert rr > 4 * REL_RMS[torch.bfloat16], (name, rr)
        assert np.abs(bad - ref).max() < 2e-2, name     # the max-abs bar alone misses it
