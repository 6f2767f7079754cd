"""GPU key-coverage checks at the benchmarked sizes, through the C ABI.

K = 0 and V an integer pattern make every visible key's weight exactly 1,
so the output must be the exact mean of V over the visible keys, bit for
bit (tests/coverage.py explains why the kernels reach it exactly).  Unlike a
tolerance on random inputs, this sees one skipped, repeated or shifted key
in any output row, at every size, in the launch configuration the benchmark
times (same shapes, so the same key splits, rotated key walk, paged pieces
and tile schedule).  Each workload is checked with fp32 output (the exact
mean) and with the input type's output (the benchmarked kernel instance).
"Every visible key" is step 3 of the *Step-by-Step Approach* of
"28. Grouped-Query Attention (GQA)": the softmax runs over all of them."""

import sys

import numpy as np
import pytest
import torch

import grouped_query_attention_fwd_amd as gqa
import workloads
from tests import coverage

pytestmark = pytest.mark.gpu

DECODES = ["decode_mistral7b_m4096", "decode_llama70b_m32768", "decode_mistral7b_m4096_fp16",
           "decode_h64_g1_m4096", "decode_h64_g16_m4096", "decode_h64_g32_m4096",
           "decode_h64_g64_m4096"]
PREFILLS = ["prefill_causal_n4096", "prefill_causal_n4096_fp16", "prefill_window4096_n16384",
            "prefill_chunk512_m4096", "prefill_causal_n4096_d256"]
PAGED = ["decode_paged_mistral7b_varlen", "decode_paged_mistral7b_full"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _outs(dtype):
    return [torch.float32] if dtype == torch.float32 else [torch.float32, dtype]


@pytest.mark.parametrize("name", DECODES)
def test_key_coverage_decode(name):
    w = workloads.by_name(name)
    say(f"key coverage {name}")
    q, k, v = workloads.key_coverage_inputs(w.B, w.H, w.H_kv, 1, w.M, w.D, w.torch_dtype)
    lo = np.zeros((w.B, 1), dtype=np.int64)
    hi = np.full((w.B, 1), w.M, dtype=np.int64)
    want = coverage.exact_means(v, w.H, lo, hi)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    del k, v
    for od in _outs(w.torch_dtype):
        out = gqa.decode(qd, kd, vd, out_dtype=od)
        torch.cuda.synchronize()
        coverage.assert_exact(out, want, f"{name} out={od}")


def test_key_coverage_decode_masked_lengths():
    """The Mistral-7B-shaped decode with a [B,1,M] mask that keeps a
    different prefix of the keys per batch row (the masked kernel instance)."""
    B, H, H_kv, M, D = 16, 32, 8, 4096, 128
    q, k, v = workloads.key_coverage_inputs(B, H, H_kv, 1, M, D, torch.bfloat16)
    lens = torch.tensor([1, 2, 15, 16, 17, 127, 128, 129, 1000, 2047, 2048, 2049, 3000, 4000,
                         4095, 4096])
    mask = (torch.arange(M)[None, :] < lens[:, None])[:, None, :].contiguous()
    lo = np.zeros((B, 1), dtype=np.int64)
    want = coverage.exact_means(v, H, lo, lens.numpy().astype(np.int64)[:, None])
    qd, kd, vd, md = q.cuda(), k.cuda(), v.cuda(), mask.cuda()
    for od in (torch.float32, torch.bfloat16):
        out = gqa.decode(qd, kd, vd, md, out_dtype=od)
        torch.cuda.synchronize()
        coverage.assert_exact(out, want, f"masked lengths out={od}")


def test_key_coverage_decode_many_splits():
    """One batch row over 65536 keys: 4 units of 64 key splits each, merged
    eight splits per round trip."""
    B, H, H_kv, M, D = 1, 16, 4, 65536, 128
    q, k, v = workloads.key_coverage_inputs(B, H, H_kv, 1, M, D, torch.bfloat16)
    want = coverage.exact_means(v, H, np.zeros((1, 1), np.int64), np.full((1, 1), M, np.int64))
    out = gqa.decode(q.cuda(), k.cuda(), v.cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    coverage.assert_exact(out, want, "65536 keys")


@pytest.mark.parametrize("name", PAGED)
def test_key_coverage_paged(name):
    w = workloads.paged_by_name(name)
    say(f"key coverage {name}")
    q, kp, vp, table, lens = workloads.key_coverage_paged(w)
    want = coverage.paged_exact_means(q.shape, kp, vp, table, lens)
    dev = [t.cuda() for t in (q, kp, vp, table, lens)]
    for od in _outs(w.torch_dtype):
        out = gqa.decode_paged(*dev, out_dtype=od)
        torch.cuda.synchronize()
        coverage.assert_exact(out, want, f"{name} out={od}")


@pytest.mark.parametrize("name", PREFILLS)
def test_key_coverage_prefill(name):
    w = workloads.by_name(name)
    say(f"key coverage {name}")
    q, k, v = workloads.key_coverage_inputs(w.B, w.H, w.H_kv, w.N, w.M, w.D, w.torch_dtype)
    band = w.band if w.band is not None else (0, -1, 0 if w.causal else -1)
    lo, hi = coverage.band_ranges(w.N, w.M, *band)
    want = coverage.exact_means(v, w.H, np.tile(lo, (w.B, 1)), np.tile(hi, (w.B, 1)))
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    del k, v
    for od in _outs(w.torch_dtype):
        if w.band is not None:
            out = gqa.prefill_band(qd, kd, vd, None, *w.band, out_dtype=od)
        else:
            out = gqa.prefill(qd, kd, vd, causal=w.causal, out_dtype=od)
        torch.cuda.synchronize()
        coverage.assert_exact(out, want, f"{name} out={od}")
