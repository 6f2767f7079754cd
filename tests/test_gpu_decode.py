"""GPU parity of gqa_decode against the fp64 oracle (through the C ABI)."""

import sys

import numpy as np
import pytest
import torch

import grouped_query_attention_fwd_amd as gqa
import workloads
from tests.parity import TOL, compare, np64, oracle_out, to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_case(seed, B, H, H_kv, M, D, dtype, mask_kind=None, q_scale=1.0, out_dtype=None):
    say(f"decode case seed={seed} B={B} H={H} H_kv={H_kv} M={M} D={D} {dtype} mask={mask_kind}")
    q, k, v, mask = workloads.random_case(seed, B, H, H_kv, 1, M, D, dtype, mask_kind, q_scale)
    ref = oracle_out(q, k, v, mask)
    qd, kd, vd, md = to_dev(q, k, v, mask)
    out = gqa.decode(qd, kd, vd, md, out_dtype=out_dtype)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    return compare(out, ref, tol, f"decode seed={seed}")


SMALL = [
    # seed, B, H, H_kv, M, D, dtype, mask
    (1, 2, 8, 2, 64, 128, torch.bfloat16, None),
    (2, 3, 8, 8, 1, 64, torch.bfloat16, None),        # MHA, single key
    (3, 2, 6, 3, 255, 32, torch.bfloat16, None),      # ragged M, g = 2
    (4, 1, 16, 1, 1000, 128, torch.bfloat16, None),   # MQA g = 16
    (5, 2, 40, 2, 777, 64, torch.bfloat16, None),     # g = 20: two head chunks
    (6, 2, 64, 1, 300, 256, torch.bfloat16, None),    # g = 64, D = 256
    (7, 4, 8, 2, 4097, 96, torch.bfloat16, None),     # D padded to 128
    (8, 2, 4, 2, 513, 8, torch.bfloat16, None),
    (9, 2, 4, 2, 130, 24, torch.bfloat16, None),
    (10, 2, 8, 2, 600, 128, torch.bfloat16, "padding"),
    (11, 2, 8, 4, 333, 128, torch.bfloat16, "random"),
    (12, 2, 8, 2, 1100, 128, torch.bfloat16, "blocks"),
    (20, 2, 8, 2, 64, 16, torch.float32, None),
    (21, 2, 4, 2, 5, 4, torch.float32, None),
    (22, 2, 12, 4, 300, 12, torch.float32, None),
    (23, 1, 16, 2, 2000, 64, torch.float32, "padding"),
    (24, 2, 8, 8, 257, 128, torch.float32, "random"),
    (25, 1, 4, 1, 700, 256, torch.float32, None),
    (26, 2, 6, 2, 1500, 36, torch.float32, "blocks"),
    (40, 2, 8, 2, 600, 128, torch.float16, None),         # fp16
    (41, 2, 40, 2, 777, 64, torch.float16, "padding"),
    (42, 1, 4, 1, 300, 256, torch.float16, None),
    (43, 2, 6, 3, 130, 24, torch.float16, "random"),
    (44, 4, 8, 2, 4097, 96, torch.float16, None),
    # one long sequence: 4 units of 64 key splits each, merged eight splits
    # per round trip
    (45, 1, 16, 4, 65536, 128, torch.bfloat16, None),
    (46, 1, 8, 1, 40000, 64, torch.float32, "padding"),   # 1 unit, 157 splits
    # 17 ... 32 heads per KV head: two head-chunk units per KV head
    (47, 2, 34, 2, 1000, 128, torch.bfloat16, None),      # g = 17: chunks of 9 and 8
    (50, 3, 64, 2, 2048, 128, torch.bfloat16, "blocks"),  # g = 32
    # more than 32 heads per KV head: the prefill-kernel path with key splits
    (48, 2, 48, 1, 800, 128, torch.float16, "random"),    # g = 48
    (49, 1, 40, 1, 5000, 64, torch.float32, "padding"),   # g = 40, fp32
    (51, 2, 128, 1, 1500, 128, torch.bfloat16, None),
    (52, 1, 96, 1, 700, 64, torch.float32, "padding"),
    (53, 1, 160, 2, 3000, 128, torch.float16, None),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"s{c[0]}")
def test_decode_small(case):
    seed, B, H, H_kv, M, D, dtype, mk = case
    run_case(seed, B, H, H_kv, M, D, dtype, mk)


def test_decode_peaky_scores():
    # q scaled x4 makes one key dominate and stresses the running-max rescale
    run_case(30, 2, 8, 2, 3000, 128, torch.bfloat16, None, q_scale=4.0)
    run_case(31, 2, 8, 2, 3000, 64, torch.float32, None, q_scale=4.0)
    run_case(33, 2, 8, 2, 3000, 128, torch.float16, None, q_scale=4.0)


def test_decode_fp32_output_of_bf16_inputs():
    mx, _ = run_case(32, 2, 8, 2, 1024, 128, torch.bfloat16, None, out_dtype=torch.float32)
    assert mx < 5e-3


def test_decode_empty_rows_are_nan():
    B, H, H_kv, M, D = 3, 8, 2, 300, 128
    q, k, v, _ = workloads.random_case(40, B, H, H_kv, 1, M, D, torch.bfloat16)
    mask = torch.ones(B, 1, M, dtype=torch.bool)
    mask[1] = False                      # batch row 1 sees nothing
    mask[2, 0, 200:] = False
    ref = oracle_out(q, k, v, mask)
    assert np.isnan(ref[1]).all()
    qd, kd, vd, md = to_dev(q, k, v, mask)
    out = gqa.decode(qd, kd, vd, md)
    compare(out, ref, TOL[torch.bfloat16], "empty rows")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("shape", [(2, 8, 2, 4096, 128), (1, 48, 3, 999, 64), (2, 4, 4, 70, 32),
                                   (2, 64, 2, 777, 128), (1, 64, 1, 3000, 64),
                                   (2, 34, 2, 500, 128), (1, 128, 1, 999, 64)])
def test_decode_head_mapping_bit_exact(dtype, shape):
    """K = 0 and V[b, j] = j: every score is 0, every weight 1, so query head
    h must return exactly h // g (repeat-interleave, not tiling)."""
    B, H, H_kv, M, D = shape
    say(f"head mapping {shape} {dtype}")
    g = H // H_kv
    q = torch.randn(B, H, 1, D).to(dtype)
    k = torch.zeros(B, H_kv, M, D, dtype=dtype)
    v = torch.arange(H_kv, dtype=torch.float32)[None, :, None, None].expand(B, H_kv, M, D)
    v = v.contiguous().to(dtype)
    qd, kd, vd = to_dev(q, k, v)
    out = gqa.decode(qd, kd, vd).float().cpu()
    want = (torch.arange(H) // g).float()[None, :, None, None].expand(B, H, 1, D)
    assert torch.equal(out, want)


def test_decode_deterministic_and_workspace_reuse():
    B, H, H_kv, M, D = 4, 32, 8, 4096, 128
    q, k, v, _ = workloads.random_case(50, B, H, H_kv, 1, M, D, torch.bfloat16)
    qd, kd, vd = to_dev(q, k, v)
    ws = torch.zeros(gqa.decode_workspace_size(B, H, H_kv, M, D), dtype=torch.uint8, device="cuda")
    outs = [gqa.decode(qd, kd, vd, workspace=ws).clone() for _ in range(5)]
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    # a different problem through the same workspace, then the first again
    q2, k2, v2, _ = workloads.random_case(51, B, H, H_kv, 1, 1000, D, torch.bfloat16)
    gqa.decode(*to_dev(q2, k2, v2), workspace=ws)
    assert torch.equal(gqa.decode(qd, kd, vd, workspace=ws), outs[0])
    compare(outs[0], oracle_out(q, k, v), TOL[torch.bfloat16], "reuse")
    torch.cuda.synchronize()
    assert ws[:gqa.DECODE_COUNTER_BYTES].count_nonzero().item() == 0


def test_decode_one_shot_calls_on_two_streams():
    """decode() without a workspace keeps one zeroed buffer per stream:
    calls queued on two streams at once use different buffers and both give
    the result of a call with a fresh workspace; a larger call on the same
    stream then replaces that stream's buffer."""
    say("one-shot decode on two streams")
    B, H, H_kv, M, D = 4, 32, 8, 4096, 128
    ins = [to_dev(*workloads.random_case(70 + i, B, H, H_kv, 1, M, D, torch.bfloat16)[:3])
           for i in range(2)]
    want = [gqa.decode(*x, workspace=torch.zeros(gqa.decode_workspace_size(B, H, H_kv, M, D),
                                                 dtype=torch.uint8, device="cuda")).clone()
            for x in ins]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[], []]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(4):
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                outs[i].append(gqa.decode(*ins[i]))
    torch.cuda.synchronize()
    for i in range(2):
        for o in outs[i]:
            assert torch.equal(o, want[i]), i
    # a call with more partials (100 units x 3 splits) grows the first
    # stream's buffer; results stay exact
    n_big = gqa.decode_workspace_size(25, 16, 4, 4096, D)
    assert n_big > gqa.decode_workspace_size(B, H, H_kv, M, D)
    q3, k3, v3 = to_dev(*workloads.random_case(72, 25, 16, 4, 1, 4096, D, torch.bfloat16)[:3])
    big = gqa.decode(q3, k3, v3, workspace=torch.zeros(n_big, dtype=torch.uint8,
                                                       device="cuda")).clone()
    with torch.cuda.stream(streams[0]):
        got_big = gqa.decode(q3, k3, v3)
        got_small = gqa.decode(*ins[0])
    torch.cuda.synchronize()
    assert torch.equal(got_big, big)
    assert torch.equal(got_small, want[0])


@pytest.mark.parametrize("B,H,H_kv,M,dtype,mask_kind", [
    (3, 128, 2, 2500, torch.bfloat16, None),      # 40 key splits per block of 64 heads
    (2, 96, 2, 1000, torch.float16, None),        # 48 heads: a block of 48 rows, 16 splits
    (2, 64, 1, 777, torch.bfloat16, "padding"),   # ragged keys, masked
    (4, 80, 2, 4096, torch.bfloat16, None),       # 40 heads per KV head
])
def test_decode_large_group_in_kernel_merge(B, H, H_kv, M, dtype, mask_kind):
    """Groups of more than 32 heads (16-bit, D = 128) run as a prefill over
    the group's heads whose key splits merge their partials among themselves
    in the same launch; every output against the oracle, twice in a row on
    one workspace (the counter area is zero after each call)."""
    say(f"large-group merge B={B} H={H} H_kv={H_kv} M={M} {dtype} mask={mask_kind}")
    q, k, v, mask = workloads.random_case(70 + B + H, B, H, H_kv, 1, M, 128, dtype, mask_kind)
    ref = oracle_out(q, k, v, mask)
    qd, kd, vd, md = to_dev(q, k, v, mask)
    n = gqa.decode_workspace_size(B, H, H_kv, M, 128)
    assert n > gqa.DECODE_COUNTER_BYTES
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    first = None
    for rep in range(2):
        out = gqa.decode(qd, kd, vd, md, workspace=ws)
        torch.cuda.synchronize()
        compare(out, ref, TOL[dtype], f"large group rep={rep}")
        assert ws[:gqa.DECODE_COUNTER_BYTES].count_nonzero().item() == 0, rep
        if first is None:
            first = out.clone()
        else:
            assert torch.equal(out, first)


def test_decode_workspace_shared_across_shapes_and_entry_points():
    """One workspace serves decode calls of different shapes, the
    large-group path and the paged form in turn: each call leaves the
    counter area zero, and what lies behind it needs no initialisation
    (it is filled with 0xFF before every call here), so every result equals
    the one from a fresh zeroed workspace."""
    say("workspace shared across shapes")
    cases = [(2, 32, 8, 4096, 128, torch.bfloat16), (1, 64, 1, 3000, 64, torch.bfloat16),
             (3, 12, 4, 777, 128, torch.float16), (2, 8, 2, 5000, 32, torch.float32),
             (16, 32, 8, 4096, 128, torch.bfloat16),
             # large groups whose key splits merge in the same launch (go and
             # claim words inside the 0xFF-filled partials): 40 and 16 splits
             (3, 128, 2, 2500, 128, torch.bfloat16), (2, 96, 2, 1000, 128, torch.float16)]
    sizes = [gqa.decode_workspace_size(B, H, Hk, M, D) for B, H, Hk, M, D, _ in cases]
    qp, kpool, vpool, table, kl = workloads.random_paged_case(53, 4, 32, 8, 128, 16, 3000,
                                                              torch.bfloat16)
    paged = [t.cuda() for t in (qp, kpool, vpool, table, kl)]
    sizes.append(gqa.decode_paged_workspace_size(4, 32, 8, table.shape[1], 16, 128))
    assert min(sizes) > 0
    ws = torch.zeros(max(sizes), dtype=torch.uint8, device="cuda")
    inputs = [to_dev(*workloads.random_case(60 + i, B, H, Hk, 1, M, D, dt)[:3])
              for i, (B, H, Hk, M, D, dt) in enumerate(cases)]
    fresh = [gqa.decode(*x, workspace=torch.zeros(n, dtype=torch.uint8, device="cuda")).clone()
             for x, n in zip(inputs, sizes)]
    fresh_paged = gqa.decode_paged(*paged, workspace=torch.zeros(sizes[-1], dtype=torch.uint8,
                                                                 device="cuda")).clone()
    nc = gqa.DECODE_COUNTER_BYTES
    for rep in range(2):
        for i in [4, 0, 5, 1, 2, 6, 3] if rep == 0 else [3, 6, 1, 0, 5, 4, 2]:
            ws[nc:].fill_(0xFF)
            assert torch.equal(gqa.decode(*inputs[i], workspace=ws), fresh[i]), (rep, i)
            torch.cuda.synchronize()
            assert ws[:nc].count_nonzero().item() == 0, (rep, i)
        ws[nc:].fill_(0xFF)
        assert torch.equal(gqa.decode_paged(*paged, workspace=ws), fresh_paged), rep
        torch.cuda.synchronize()
        assert ws[:nc].count_nonzero().item() == 0, rep


def test_decode_mistral7b_full():
    """Mistral-7B-shaped decode at full size, every output checked."""
    w = workloads.by_name("decode_mistral7b_m4096")
    q, k, v, mask, _ = workloads.make_inputs(w)
    say("decode mistral full")
    out = gqa.decode(*to_dev(q, k, v))
    mx, rr = compare(out, oracle_out(q, k, v), TOL[torch.bfloat16], w.name)
    say(f"  max abs err {mx:.3e} rel rms {rr:.3e}")


def test_decode_llama70b_full():
    """Llama-2-70B-shaped decode (M = 32768) at full size, in the launch
    configuration the benchmark times; every output of all 16 batch rows
    checked against the oracle (which computes them one batch row at a
    time: batch rows are independent in the definition)."""
    w = workloads.by_name("decode_llama70b_m32768")
    q, k, v, mask, _ = workloads.make_inputs(w)
    say("decode llama70b full")
    out = gqa.decode(*to_dev(q, k, v)).cpu()
    for b in range(w.B):
        ref = oracle_out(q[b:b + 1], k[b:b + 1], v[b:b + 1])
        mx, rr = compare(out[b:b + 1], ref, TOL[torch.bfloat16], f"{w.name} b={b}")
        say(f"  b={b} max abs err {mx:.3e} rel rms {rr:.3e}")


@pytest.mark.parametrize("name", [w.name for w in workloads.GROUP_SWEEP])
def test_decode_group_sweep_sampled(name):
    """The group-size sweep (64 query heads, g = 1 ... 64) at full size in
    the benchmarked launch configuration; two batch rows against the oracle."""
    w = workloads.by_name(name)
    q, k, v, _, _ = workloads.make_inputs(w)
    say(f"decode group sweep {name}")
    out = gqa.decode(*to_dev(q, k, v)).cpu()
    for b in (0, w.B - 1):
        ref = oracle_out(q[b:b + 1], k[b:b + 1], v[b:b + 1])
        compare(out[b:b + 1], ref, TOL[torch.bfloat16], f"{name} b={b}")


def test_decode_mistral7b_fp16_full():
    """The headline decode shape with fp16 inputs, every output element."""
    w = workloads.by_name("decode_mistral7b_m4096_fp16")
    q, k, v, mask, _ = workloads.make_inputs(w)
    say("decode mistral7b fp16 full")
    out = gqa.decode(*to_dev(q, k, v))
    mx, rr = compare(out, oracle_out(q, k, v), TOL[torch.float16], w.name)
    say(f"  max abs err {mx:.3e} rel rms {rr:.3e}")


def test_decode_grid_of_more_than_65536_workgroups():
    """8200 batch rows of 8 KV heads (g = 1): 65,600 units, one workgroup
    each, more than one grid row holds, so the launch folds them into grid z."""
    run_case(91, 8200, 8, 8, 3, 8, torch.bfloat16)
