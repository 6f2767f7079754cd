"""GPU parity of gqa_prefill against the fp64 oracle (through the C ABI)."""

import sys

import numpy as np
import pytest
import torch

import grouped_query_attention_fwd_amd as gqa
import workloads
from tests.parity import TOL, compare, np64, oracle_out, to_dev

import oracle

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_case(seed, B, H, H_kv, N, M, D, dtype, mask_kind=None, causal=False, q_scale=1.0,
             out_dtype=None):
    say(f"prefill case seed={seed} B={B} H={H} H_kv={H_kv} N={N} M={M} D={D} {dtype} "
        f"mask={mask_kind} causal={causal}")
    q, k, v, mask = workloads.random_case(seed, B, H, H_kv, N, M, D, dtype, mask_kind, q_scale)
    ref = oracle_out(q, k, v, mask, causal)
    qd, kd, vd, md = to_dev(q, k, v, mask)
    out = gqa.prefill(qd, kd, vd, md, causal=causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return compare(out, ref, TOL[dtype], f"prefill seed={seed}")


SMALL = [
    # seed, B, H, H_kv, N, M, D, dtype, mask, causal
    (1, 2, 8, 2, 64, 64, 128, torch.bfloat16, None, False),
    (2, 1, 8, 2, 130, 130, 128, torch.bfloat16, None, True),     # ragged, causal
    (3, 2, 4, 4, 77, 200, 64, torch.bfloat16, None, False),      # MHA, N != M
    (4, 1, 6, 3, 65, 31, 32, torch.bfloat16, None, True),        # g = 2, causal N > M
    (5, 2, 3, 1, 40, 300, 128, torch.bfloat16, None, True),      # g = 3 (HG 1), causal N < M
    (6, 1, 16, 2, 100, 100, 256, torch.bfloat16, None, True),    # D = 256
    (7, 2, 8, 2, 50, 70, 8, torch.bfloat16, "random", False),
    (8, 2, 8, 1, 90, 260, 96, torch.bfloat16, "padding", False),
    (9, 2, 8, 2, 64, 400, 128, torch.bfloat16, "blocks", False),  # skipped tiles
    (10, 2, 8, 4, 129, 129, 72, torch.bfloat16, "random", True),  # mask AND causal
    (11, 1, 4, 2, 1, 1, 128, torch.bfloat16, None, False),
    (12, 1, 4, 2, 1, 500, 128, torch.bfloat16, None, True),      # one row sees key 0 only
    (20, 1, 4, 2, 5, 5, 4, torch.float32, None, False),
    (21, 2, 8, 2, 33, 47, 24, torch.float32, "padding", False),
    (22, 1, 6, 2, 70, 70, 16, torch.float32, None, True),
    (23, 2, 4, 4, 20, 90, 64, torch.float32, "random", False),
    (24, 1, 8, 2, 40, 40, 128, torch.float32, None, True),
    (25, 1, 4, 1, 17, 33, 256, torch.float32, "blocks", False),
    (26, 2, 6, 3, 31, 200, 36, torch.float32, "random", True),
    (40, 2, 8, 2, 130, 130, 128, torch.float16, None, True),      # fp16
    (41, 1, 6, 3, 77, 200, 64, torch.float16, "padding", False),
    (42, 1, 16, 2, 100, 100, 256, torch.float16, None, True),
    (43, 2, 8, 4, 129, 129, 72, torch.float16, "random", True),
    (44, 1, 3, 1, 40, 300, 32, torch.float16, "blocks", False),
    # 256-wide 16-bit rows (eight-wave workgroups, 32-key tiles): masked,
    # g = 3 (one head per block, 128 positions), staged rows (D = 200),
    # a ragged key tail
    (45, 2, 8, 2, 150, 170, 256, torch.bfloat16, "random", False),
    (46, 1, 6, 2, 300, 300, 256, torch.bfloat16, None, True),
    (47, 1, 8, 4, 70, 90, 200, torch.float16, "padding", True),
    (48, 2, 4, 1, 33, 1000, 256, torch.bfloat16, "blocks", False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"s{c[0]}")
def test_prefill_small(case):
    seed, B, H, H_kv, N, M, D, dtype, mk, causal = case
    run_case(seed, B, H, H_kv, N, M, D, dtype, mk, causal)


def test_prefill_peaky_scores():
    run_case(30, 1, 8, 2, 200, 200, 128, torch.bfloat16, None, True, q_scale=4.0)
    run_case(32, 1, 8, 2, 200, 200, 128, torch.float16, None, True, q_scale=4.0)
    run_case(31, 1, 8, 2, 100, 150, 24, torch.float32, "padding", False, q_scale=4.0)


def test_prefill_fp32_output_of_bf16_inputs():
    mx, _ = run_case(32, 1, 8, 2, 256, 256, 128, torch.bfloat16, None, True,
                     out_dtype=torch.float32)
    assert mx < 1e-2


def test_prefill_empty_rows_are_nan():
    B, H, H_kv, N, M, D = 2, 8, 2, 40, 90, 128
    q, k, v, _ = workloads.random_case(40, B, H, H_kv, N, M, D, torch.bfloat16)
    mask = torch.rand(B, N, M, generator=torch.Generator().manual_seed(3)) < 0.5
    mask[0, 5] = False
    mask[1, 17:23] = False
    ref = oracle_out(q, k, v, mask)
    out = gqa.prefill(*to_dev(q, k, v, mask))
    compare(out, ref, TOL[torch.bfloat16], "empty rows")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("shape", [(2, 8, 2, 100, 100, 128, True), (1, 6, 2, 65, 300, 32, False),
                                   (1, 4, 4, 33, 33, 64, True), (1, 12, 1, 20, 70, 128, False)])
def test_prefill_head_mapping_bit_exact(dtype, shape):
    """K = 0 and V[b, j] = j: every visible weight is 1, so query head h must
    return exactly h // g for every position (causal or not)."""
    B, H, H_kv, N, M, D, causal = shape
    say(f"head mapping {shape} {dtype}")
    g = H // H_kv
    q = torch.randn(B, H, N, D).to(dtype)
    k = torch.zeros(B, H_kv, M, D, dtype=dtype)
    v = torch.arange(H_kv, dtype=torch.float32)[None, :, None, None].expand(B, H_kv, M, D)
    v = v.contiguous().to(dtype)
    out = gqa.prefill(*to_dev(q, k, v), causal=causal).float().cpu()
    want = (torch.arange(H) // g).float()[None, :, None, None].expand(B, H, N, D)
    assert torch.equal(out, want)


def test_prefill_deterministic():
    q, k, v, _ = workloads.random_case(50, 1, 8, 2, 300, 300, 128, torch.bfloat16)
    qd, kd, vd = to_dev(q, k, v)
    a = gqa.prefill(qd, kd, vd, causal=True)
    for _ in range(3):
        assert torch.equal(gqa.prefill(qd, kd, vd, causal=True), a)


def test_prefill_tiny_worked_example_config():
    """Tiny fp32 workload (q [1,4,5,4], k/v [1,2,5,4]) in full."""
    w = workloads.by_name("tiny_fp32")
    q, k, v, mask, causal = workloads.make_inputs(w)
    out = gqa.prefill(*to_dev(q, k, v))
    assert tuple(out.shape) == (1, 4, 5, 4)
    compare(out, oracle_out(q, k, v), TOL[torch.float32], w.name)


def test_prefill_padded_d24_full():
    """Padded fp32 prefill (B4 H32 H_kv4 N=M=512 D24, mask j < len_b) in full."""
    w = workloads.by_name("prefill_padded_d24")
    q, k, v, mask, causal = workloads.make_inputs(w)
    out = gqa.prefill(*to_dev(q, k, v, mask))
    mx, rr = compare(out, oracle_out(q, k, v, mask), TOL[torch.float32], w.name)
    say(f"  max abs err {mx:.3e} rel rms {rr:.3e}")


@pytest.mark.parametrize("name", ["prefill_causal_n4096", "prefill_causal_n4096_fp16",
                                  "prefill_causal_n4096_d256"])
def test_prefill_causal_n4096_full_sampled(name):
    """Causal prefill (B4 H32 H_kv8 N=M=4096 D128, bf16 and fp16; B2 H16
    H_kv4 D256 bf16) at full size, in the launch configuration the benchmark
    times.  Sampled query rows
    of every (batch row, head) are checked against the oracle, which evaluates
    a row i as an explicit mask j <= i (causal == that mask is an oracle pin)."""
    w = workloads.by_name(name)
    q, k, v, mask, causal = workloads.make_inputs(w)
    say("prefill causal full")
    out = gqa.prefill(*to_dev(q, k, v), causal=True).cpu()
    rows = [0, 1, 15, 16, 63, 64, 127, 1000, 2047, 2048, 3001, 4094, 4095]
    qs = q[:, :, rows, :]
    M = k.shape[2]
    m = torch.zeros(q.shape[0], len(rows), M, dtype=torch.bool)
    for r, i in enumerate(rows):
        m[:, r, : i + 1] = True
    for b in range(q.shape[0]):
        ref = oracle.gqa(np64(qs[b:b + 1]), np64(k[b:b + 1]), np64(v[b:b + 1]), np64(m[b:b + 1]))
        mx, rr = compare(out[b:b + 1, :, rows, :], ref, TOL[w.torch_dtype], f"{w.name} b={b}")
        say(f"  b={b} max abs err {mx:.3e} rel rms {rr:.3e}")


@pytest.mark.parametrize("name", ["prefill_causal_n4096", "prefill_causal_n4096_fp16"])
def test_prefill_causal_n4096_whole_groups(name):
    """The causal N = 4096 prefill at full size: every output row of four of
    its 32 (batch row, KV head) groups, one per batch row and each a
    different KV head, against the oracle run on that group alone (its g
    query heads with their one K/V head: groups are independent in the
    definition, so the slice is the same attention)."""
    w = workloads.by_name(name)
    q, k, v, mask, causal = workloads.make_inputs(w)
    say(f"prefill causal whole groups {name}")
    out = gqa.prefill(*to_dev(q, k, v), causal=True).cpu()
    g = w.H // w.H_kv
    for b, j in ((0, 0), (1, 3), (2, 5), (3, 7)):
        hs = slice(g * j, g * (j + 1))
        ref = oracle.gqa(np64(q[b:b + 1, hs]), np64(k[b:b + 1, j:j + 1]),
                         np64(v[b:b + 1, j:j + 1]), None, True)
        mx, rr = compare(out[b:b + 1, hs], ref, TOL[w.torch_dtype], f"{name} b={b} j={j}")
        say(f"  b={b} j={j} max abs err {mx:.3e} rel rms {rr:.3e}")


def test_prefill_grid_of_more_than_65536_workgroups():
    """1040 query heads (g = 1) of 4100 fp32 positions: 65 blocks of 64
    positions per head, 67,600 workgroups, more than one grid row holds, so
    the launch folds them into grid z."""
    B, H, H_kv, N, M, D = 1, 1040, 1040, 4100, 5, 4
    say("prefill folded grid")
    q, k, v, _ = workloads.random_case(90, B, H, H_kv, N, M, D, torch.float32)
    out = gqa.prefill(*to_dev(q, k, v), causal=True)
    compare(out, oracle_out(q, k, v, causal=True), TOL[torch.float32], "folded grid")
