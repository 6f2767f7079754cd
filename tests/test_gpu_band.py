"""GPU parity of gqa_prefill_band (sliding windows, bottom-right causal,
two-sided bands) against the fp64 oracle, through the C ABI."""

import sys

import numpy as np
import pytest
import torch

import grouped_query_attention_fwd_amd as gqa
import oracle
import workloads
from tests.parity import TOL, compare, np64, to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_band(seed, B, H, H_kv, N, M, D, dtype, q_off, wl, wr, mask_kind=None, out_dtype=None):
    say(f"band case seed={seed} B={B} H={H} H_kv={H_kv} N={N} M={M} D={D} {dtype} "
        f"q_offset={q_off} wl={wl} wr={wr} mask={mask_kind}")
    q, k, v, mask = workloads.random_case(seed, B, H, H_kv, N, M, D, dtype, mask_kind)
    ref = oracle.gqa_band(np64(q), np64(k), np64(v), np64(mask), q_off, wl, wr)
    qd, kd, vd, md = to_dev(q, k, v, mask)
    out = gqa.prefill_band(qd, kd, vd, md, q_off, wl, wr, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return compare(out, ref, TOL[dtype], f"band seed={seed}"), (qd, kd, vd, md, out)


SMALL = [
    # seed, B, H, H_kv, N, M, D, dtype, q_offset, window_left, window_right, mask
    (1, 2, 8, 2, 200, 200, 128, torch.bfloat16, 0, 63, 0, None),       # sliding window 64
    (2, 2, 8, 2, 100, 300, 128, torch.bfloat16, 200, -1, 0, None),     # bottom-right causal
    (3, 2, 8, 2, 300, 100, 128, torch.bfloat16, -50, -1, 0, None),     # leading rows see nothing
    (4, 2, 12, 4, 130, 257, 24, torch.float32, 5, 10, 20, None),       # two-sided band
    (5, 2, 8, 8, 257, 513, 64, torch.bfloat16, 0, -1, 31, None),       # right edge only
    (6, 1, 16, 2, 333, 333, 128, torch.bfloat16, 0, 100, 0, "padding"),
    (7, 2, 6, 2, 190, 450, 64, torch.bfloat16, 260, 37, 0, "random"),  # window + chunk + mask
    (8, 1, 4, 1, 129, 600, 256, torch.bfloat16, 471, 200, 0, None),    # D = 256
    (9, 2, 6, 3, 77, 77, 4, torch.float32, 0, 7, 3, None),             # fp32, D = 4, g = 2
    (10, 1, 8, 2, 1000, 1000, 128, torch.bfloat16, 0, 0, 0, None),     # window 1: the own key
    (11, 2, 8, 2, 64, 640, 128, torch.bfloat16, 576, 127, 0, "blocks"),
    (12, 1, 3, 1, 150, 150, 32, torch.bfloat16, 0, 31, 0, None),       # g = 3
    (13, 2, 8, 2, 300, 700, 128, torch.float16, 400, 99, 0, None),     # fp16 window + chunk
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"b{c[0]}")
def test_band_small(case):
    seed, B, H, H_kv, N, M, D, dtype, qo, wl, wr, mk = case
    run_band(seed, B, H, H_kv, N, M, D, dtype, qo, wl, wr, mk)


def test_band_fp32_output():
    (mx, _), _ = run_band(20, 2, 8, 2, 300, 300, 128, torch.bfloat16, 0, 50, 0,
                          out_dtype=torch.float32)
    assert mx < 5e-3


def test_band_causal_equals_prefill_causal_bitwise():
    """The causal entry point is the band (0, open, 0): same kernel, same bits."""
    say("band vs causal prefill")
    q, k, v, _ = workloads.random_case(21, 2, 8, 2, 300, 300, 128, torch.bfloat16)
    qd, kd, vd = to_dev(q, k, v)
    a = gqa.prefill(qd, kd, vd, causal=True)
    b = gqa.prefill_band(qd, kd, vd, None, 0, -1, 0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_band_chunk_matches_full_causal_rows():
    """A bottom-right causal chunk gives the last rows of full causal
    self-attention (up to rounding: the tiles and rescale points differ)."""
    say("chunk vs full causal")
    B, H, H_kv, M, N, D = 2, 8, 2, 700, 190, 128
    q, k, v, _ = workloads.random_case(22, B, H, H_kv, M, M, D, torch.bfloat16)
    qd, kd, vd = to_dev(q, k, v)
    full = gqa.prefill(qd, kd, vd, causal=True, out_dtype=torch.float32)
    chunk = gqa.prefill_band(qd[:, :, M - N:].contiguous(), kd, vd, None, M - N, -1, 0,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert (full[:, :, M - N:] - chunk).abs().max().item() < 2e-3


def test_band_all_rows_empty():
    """An offset that puts every query before key 0 leaves every row empty."""
    say("band with no visible key")
    q, k, v, _ = workloads.random_case(23, 1, 4, 2, 40, 50, 64, torch.bfloat16)
    qd, kd, vd = to_dev(q, k, v)
    out = gqa.prefill_band(qd, kd, vd, None, -100, -1, 0)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()


@pytest.mark.parametrize("name", ["prefill_window4096_n16384", "prefill_chunk512_m4096"])
def test_band_workload_sampled_rows(name):
    """The benchmarked banded workloads, in the launch configuration the
    benchmark uses, checked on sampled query rows (the oracle computes a row
    alone by shifting the offset)."""
    w = workloads.by_name(name)
    say(f"band workload {name}")
    q, k, v, mask, _ = workloads.make_inputs(w)
    qo, wl, wr = w.band
    qd, kd, vd = to_dev(q, k, v)
    out = gqa.prefill_band(qd, kd, vd, None, qo, wl, wr)
    torch.cuda.synchronize()
    rows = sorted({0, 1, 15, 16, 63, 64, 127, 511, w.N // 2, w.N - 2, w.N - 1} |
                  ({4095, 4096, 4097, 8191, 12000} if w.N > 8192 else set()))
    bs = [0, w.B - 1] if w.B > 1 else [0]
    for b in bs:
        kb, vb = np64(k[b:b + 1]), np64(v[b:b + 1])
        for i in rows:
            ref = oracle.gqa_band(np64(q[b:b + 1, :, i:i + 1]), kb, vb, None, qo + i, wl, wr)
            compare(out[b:b + 1, :, i:i + 1], ref, TOL[torch.bfloat16], f"{name} b={b} row={i}")


@pytest.mark.parametrize("name,b,j,r0,r1", [
    ("prefill_chunk512_m4096", 0, 0, 0, 512),         # every row of the chunk
    ("prefill_chunk512_m4096", 15, 7, 0, 512),
    ("prefill_window4096_n16384", 0, 3, 8192, 9216),  # a block of 1024 rows
    ("prefill_window4096_n16384", 0, 6, 15360, 16384),
])
def test_band_workload_whole_group_rows(name, b, j, r0, r1):
    """The benchmarked banded workloads at full size: every query row in
    [r0, r1) of the g query heads of one (batch row, KV head) group against
    the oracle run on that group alone (groups are independent in the
    definition; the rows' positions enter as the offset)."""
    w = workloads.by_name(name)
    say(f"band workload whole group {name} b={b} j={j} rows {r0}..{r1}")
    q, k, v, mask, _ = workloads.make_inputs(w)
    qo, wl, wr = w.band
    qd, kd, vd = to_dev(q, k, v)
    out = gqa.prefill_band(qd, kd, vd, None, qo, wl, wr)
    torch.cuda.synchronize()
    g = w.H // w.H_kv
    hs = slice(g * j, g * (j + 1))
    ref = oracle.gqa_band(np64(q[b:b + 1, hs, r0:r1]), np64(k[b:b + 1, j:j + 1]),
                          np64(v[b:b + 1, j:j + 1]), None, qo + r0, wl, wr)
    mx, rr = compare(out[b:b + 1, hs, r0:r1], ref, TOL[torch.bfloat16], f"{name} b={b} j={j}")
    say(f"  max abs err {mx:.3e} rel rms {rr:.3e}")
