"""GPU parity of gqa_decode_paged (paged KV cache, per-sequence lengths)
against the fp64 oracle, through the C ABI."""

import sys

import numpy as np
import pytest
import torch

import grouped_query_attention_fwd_amd as gqa
import oracle
import workloads
from tests.parity import TOL, compare, np64

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_paged(q, kp, vp, table, lens):
    return oracle.gqa_paged(np64(q), np64(kp), np64(vp), table.numpy(), lens.numpy())


def run_paged(q, kp, vp, table, lens, dtype, what, out_dtype=None, workspace=None):
    ref = oracle_paged(q, kp, vp, table, lens)
    dev = [t.cuda() for t in (q, kp, vp, table, lens)]
    out = gqa.decode_paged(*dev, out_dtype=out_dtype, workspace=workspace)
    torch.cuda.synchronize()
    tol = TOL[torch.float32] if out_dtype == torch.float32 and dtype == torch.float32 \
        else TOL[dtype]
    return compare(out, ref, tol, what), out


SMALL = [
    # seed, B, H, H_kv, D, block_size, max_len, dtype, lengths
    (1, 4, 8, 2, 128, 16, 100, torch.bfloat16, "uniform"),
    (2, 6, 8, 2, 64, 32, 70, torch.float32, [0, 1, 31, 32, 33, 64]),
    (3, 3, 8, 8, 128, 16, 300, torch.bfloat16, "uniform"),     # MHA
    (4, 2, 16, 1, 128, 64, 1000, torch.bfloat16, "uniform"),   # MQA g = 16
    (5, 2, 40, 2, 64, 16, 777, torch.bfloat16, "full"),        # g = 20: two head chunks
    (6, 2, 64, 1, 256, 32, 300, torch.bfloat16, "uniform"),    # g = 64, D = 256
    (7, 3, 8, 2, 96, 16, 4097, torch.bfloat16, [4097, 2500, 17]),  # D padded, splits
    (8, 2, 12, 4, 24, 48, 500, torch.float32, "uniform"),      # fp32, D = 24
    (9, 2, 4, 2, 16, 16, 200, torch.float32, "full"),          # fp32, D = 16
    (10, 2, 8, 2, 128, 256, 1000, torch.bfloat16, [1000, 999]),  # large blocks
    (11, 5, 32, 8, 128, 16, 5000, torch.bfloat16, "uniform"),  # several splits
    (12, 2, 4, 2, 256, 16, 700, torch.float32, "uniform"),     # fp32 D = 256
    (13, 4, 32, 8, 128, 16, 3000, torch.float16, "uniform"),   # fp16
    (14, 5, 64, 2, 128, 16, 2500, torch.bfloat16, "uniform"),  # g = 32: two head chunks
    (15, 3, 48, 1, 64, 32, 1500, torch.float32, [1500, 3, 700]),  # g = 48, fp32: three chunks
    (16, 2, 128, 1, 128, 16, 900, torch.bfloat16, "uniform"),  # g = 128: eight head chunks
]


# Length-balanced pieces: at most 256 workgroups, the longest piece as short
# as the lengths allow, each unit cut into near-equal pieces.
BALANCED = [
    # seed, B, H, H_kv, D, block_size, max_len, dtype, lengths
    (30, 8, 64, 8, 128, 16, 4096, torch.bfloat16, [4096, 0, 0, 0, 0, 0, 0, 1]),  # one long row
    (31, 31, 64, 8, 128, 16, 700, torch.bfloat16, "uniform"),   # 248 units: 8 spare workgroups
    (32, 1, 32, 8, 128, 16, 5000, torch.bfloat16, "full"),      # 8 units, 32 pieces each
    (33, 3, 72, 3, 64, 32, 2000, torch.bfloat16, [2000, 1, 1000]),  # g = 24: two head chunks
    (34, 4, 16, 4, 128, 16, 900, torch.bfloat16, [0, 0, 0, 0]),  # no keys anywhere: NaN
    (35, 5, 20, 5, 128, 64, 3000, torch.float16, [3000, 64, 65, 2999, 128]),
    (36, 2, 8, 2, 32, 16, 6000, torch.float32, [6000, 17]),     # fp32, many pieces
    # 320 units (more than one wave of workgroups): 640 workgroups
    (37, 40, 16, 8, 64, 16, 700, torch.bfloat16, "uniform"),   # uneven: balanced pieces
    (38, 40, 16, 8, 64, 16, 700, torch.bfloat16, "full"),      # even: one piece per unit
    (39, 36, 16, 8, 64, 32, 1000, torch.float16, [1000] * 35 + [3]),  # near-even but one short
]


@pytest.mark.parametrize("case", BALANCED, ids=lambda c: f"b{c[0]}")
def test_paged_balanced_pieces(case):
    seed, B, H, H_kv, D, bs, max_len, dtype, lens = case
    say(f"paged balanced case seed={seed} B={B} H={H} H_kv={H_kv} D={D} bs={bs} "
        f"max_len={max_len} {dtype} lens={lens if isinstance(lens, str) else lens}")
    q, kp, vp, table, kl = workloads.random_paged_case(seed, B, H, H_kv, D, bs, max_len,
                                                       dtype, lengths=lens)
    run_paged(q, kp, vp, table, kl, dtype, f"paged balanced {seed}")


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"p{c[0]}")
def test_paged_small(case):
    seed, B, H, H_kv, D, bs, max_len, dtype, lens = case
    say(f"paged case seed={seed} B={B} H={H} H_kv={H_kv} D={D} bs={bs} max_len={max_len} "
        f"{dtype} lens={lens}")
    q, kp, vp, table, kl = workloads.random_paged_case(seed, B, H, H_kv, D, bs, max_len,
                                                       dtype, lengths=lens)
    run_paged(q, kp, vp, table, kl, dtype, f"paged seed={seed}")


def test_paged_shared_block_and_fp32_out():
    say("paged shared first block, fp32 output")
    q, kp, vp, table, kl = workloads.random_paged_case(
        20, 3, 8, 2, 128, 16, 600, torch.bfloat16, lengths=[600, 450, 33],
        shared_first_block=True)
    assert table[1, 0] == table[0, 0]
    (mx, _), _ = run_paged(q, kp, vp, table, kl, torch.bfloat16, "paged shared",
                           out_dtype=torch.float32)
    assert mx < 5e-3


def test_paged_peaky_scores():
    say("paged peaky scores")
    q, kp, vp, table, kl = workloads.random_paged_case(21, 2, 8, 2, 128, 32, 3000,
                                                       torch.bfloat16, q_scale=4.0)
    run_paged(q, kp, vp, table, kl, torch.bfloat16, "paged peaky")


def test_paged_length_clamping():
    """kv_len above max_blocks*block_size counts as full; a negative or zero
    length sees no key (NaN row)."""
    say("paged length clamping")
    B, H, H_kv, D, bs, L = 3, 8, 2, 64, 16, 160
    q, kp, vp, table, kl = workloads.random_paged_case(22, B, H, H_kv, D, bs, L,
                                                       torch.bfloat16, lengths=[L, L, 0])
    dev = [t.cuda() for t in (q, kp, vp, table)]
    weird = torch.tensor([L + 1000, -7, 0], dtype=torch.int32, device="cuda")
    out = gqa.decode_paged(*dev, weird)
    torch.cuda.synchronize()
    ref = oracle.gqa_paged(np64(q), np64(kp), np64(vp), table.numpy(), np.array([L, 0, 0]))
    compare(out, ref, TOL[torch.bfloat16], "paged clamp")
    assert torch.isnan(out[1:]).all()


def test_paged_matches_contiguous_decode_full_lengths():
    """With every sequence full, the paged call computes what gqa_decode
    computes on the gathered cache.  The two cut the keys into different
    pieces (the paged call balances them over the actual lengths), so they
    agree to rounding, and each is bit-reproducible."""
    say("paged vs contiguous, full lengths")
    B, H, H_kv, D, bs, L = 4, 32, 8, 128, 16, 2048
    q, kp, vp, table, kl = workloads.random_paged_case(23, B, H, H_kv, D, bs, L,
                                                       torch.bfloat16, lengths="full")
    qd, kpd, vpd, td, kld = [t.cuda() for t in (q, kp, vp, table, kl)]
    # gather [B, max_blocks] blocks -> [B, max_blocks, H_kv, bs, D] -> [B, H_kv, L, D]
    kc = kpd[td.long()].permute(0, 2, 1, 3, 4).reshape(B, H_kv, L, D).contiguous()
    vc = vpd[td.long()].permute(0, 2, 1, 3, 4).reshape(B, H_kv, L, D).contiguous()
    a = gqa.decode(qd, kc, vc, out_dtype=torch.float32)
    b = gqa.decode_paged(qd, kpd, vpd, td, kld, out_dtype=torch.float32)
    b2 = gqa.decode_paged(qd, kpd, vpd, td, kld, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(b, b2)
    diff = (a - b).abs().max().item()
    say(f"  max |contiguous - paged| = {diff:.3e}")
    assert diff <= 1e-3      # fp32 outputs; only the merge points differ


def test_paged_matches_masked_decode():
    """Mixed lengths: equal to gqa_decode over the gathered cache with the
    length mask (which reads every key and hides the tail)."""
    say("paged vs masked contiguous, mixed lengths")
    B, H, H_kv, D, bs, L = 5, 16, 4, 128, 32, 1500
    q, kp, vp, table, kl = workloads.random_paged_case(24, B, H, H_kv, D, bs, L,
                                                       torch.bfloat16)
    tfull = table.clone()
    nb = kp.shape[0]
    tfull[tfull < 0] = 0                     # any valid block for the hidden tail
    qd, kpd, vpd, td, kld = [t.cuda() for t in (q, kp, vp, table, kl)]
    mb = table.shape[1]
    M = mb * bs
    idx = tfull.long().cuda()
    assert int(idx.max()) < nb
    kc = kpd[idx].permute(0, 2, 1, 3, 4).reshape(B, H_kv, M, D).contiguous()
    vc = vpd[idx].permute(0, 2, 1, 3, 4).reshape(B, H_kv, M, D).contiguous()
    mask = (torch.arange(M, device="cuda")[None, :] < kld[:, None].long())[:, None, :]
    a = gqa.decode(qd, kc, vc, mask.contiguous())
    b = gqa.decode_paged(qd, kpd, vpd, td, kld)
    torch.cuda.synchronize()
    diff = (a.float() - b.float()).abs().max().item()
    say(f"  max |masked - paged| = {diff:.3e}, identical={torch.equal(a, b)}")
    assert diff <= 1e-2


def test_paged_determinism_and_workspace_reuse():
    say("paged determinism")
    q, kp, vp, table, kl = workloads.random_paged_case(25, 4, 32, 8, 128, 16, 4096,
                                                       torch.bfloat16)
    dev = [t.cuda() for t in (q, kp, vp, table, kl)]
    need = gqa.decode_paged_workspace_size(4, 32, 8, table.shape[1], 16, 128)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    op = gqa.decode_paged_op(*dev, workspace=ws)
    a = op().clone()
    torch.cuda.synchronize()
    nc = gqa.DECODE_COUNTER_BYTES
    assert ws[:nc].count_nonzero().item() == 0   # the call leaves its counters zero
    ws[nc:].fill_(0xFF)                          # the partials need no initialisation
    b = op().clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("name", [w.name for w in workloads.PAGED_WORKLOADS])
def test_paged_workload_full_size(name):
    """The benchmarked paged workloads, every output element."""
    w = workloads.paged_by_name(name)
    say(f"paged workload {name}")
    q, kp, vp, table, kl = workloads.make_paged_inputs(w)
    (mx, rr), _ = run_paged(q, kp, vp, table, kl, w.torch_dtype, name)
    say(f"  max abs err {mx:.3e}, rel rms {rr:.2e}")
