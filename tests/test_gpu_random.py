"""Seeded random-shape parity sweep over every entry point and dtype: each
case draws its sizes, group, head dim, dtype, mask and band from a fixed
seed, runs the HIP path through the C ABI and compares with the oracle."""

import os
import random
import sys

import numpy as np
import pytest
import torch

import grouped_query_attention_fwd_amd as gqa
import oracle
import workloads
from tests.parity import TOL, compare, np64, to_dev

pytestmark = pytest.mark.gpu

DTYPES = [torch.bfloat16, torch.float16, torch.float32]
# cases per entry point (a longer sweep: GQA_RANDOM_CASES=200)
CASES = int(os.environ.get("GQA_RANDOM_CASES", "12"))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def draw_shape(r, dtype):
    g = r.choice([1, 2, 3, 4, 5, 8, 16, 24, 32, 40, 64])
    # the oracle materialises the repeated K/V: keep H = g * H_kv modest
    H_kv = r.choice([1, 2, 3, 4, 8] if g <= 16 else [1, 2])
    if dtype == torch.float32:
        D = r.choice([4, 8, 12, 16, 24, 32, 40, 64, 100, 128, 256])
    else:
        D = r.choice([8, 16, 24, 32, 48, 64, 96, 128, 136, 256])
    return r.randint(1, 3), g * H_kv, H_kv, D


@pytest.mark.parametrize("seed", range(CASES))
def test_random_decode(seed):
    r = random.Random(1000 + seed)
    dtype = DTYPES[seed % 3]
    B, H, H_kv, D = draw_shape(r, dtype)
    M = r.choice([1, 7, 64, 255, 256, 257, 1000, 2048, 3333])
    mk = r.choice([None, None, "padding", "random", "blocks"])
    say(f"random decode seed={seed} B={B} H={H} H_kv={H_kv} M={M} D={D} {dtype} mask={mk}")
    q, k, v, mask = workloads.random_case(2000 + seed, B, H, H_kv, 1, M, D, dtype, mk)
    ref = oracle.gqa(np64(q), np64(k), np64(v), np64(mask))
    out = gqa.decode(*to_dev(q, k, v, mask))
    torch.cuda.synchronize()
    compare(out, ref, TOL[dtype], f"random decode {seed}")


@pytest.mark.parametrize("seed", range(CASES))
def test_random_prefill_band(seed):
    r = random.Random(3000 + seed)
    dtype = DTYPES[seed % 3]
    B, H, H_kv, D = draw_shape(r, dtype)
    N = r.choice([1, 5, 31, 64, 65, 130, 257])
    M = r.choice([1, 9, 64, 100, 255, 300])
    mk = r.choice([None, None, "padding", "random"])
    q_off = r.choice([0, 0, M - N, r.randint(-20, 40)])
    wl = r.choice([-1, -1, 0, 7, 63])
    wr = r.choice([-1, 0, 0, 5])
    say(f"random band seed={seed} B={B} H={H} H_kv={H_kv} N={N} M={M} D={D} {dtype} "
        f"mask={mk} band=({q_off},{wl},{wr})")
    q, k, v, mask = workloads.random_case(4000 + seed, B, H, H_kv, N, M, D, dtype, mk)
    ref = oracle.gqa_band(np64(q), np64(k), np64(v), np64(mask), q_off, wl, wr)
    qd, kd, vd, md = to_dev(q, k, v, mask)
    out = gqa.prefill_band(qd, kd, vd, md, q_off, wl, wr)
    torch.cuda.synchronize()
    compare(out, ref, TOL[dtype], f"random band {seed}")


@pytest.mark.parametrize("seed", range(max(8, CASES * 2 // 3)))
def test_random_paged(seed):
    r = random.Random(5000 + seed)
    dtype = DTYPES[seed % 3]
    B, H, H_kv, D = draw_shape(r, dtype)
    bs = r.choice([16, 32, 48, 64, 256])
    max_len = r.choice([1, 16, 100, 1000, 2500])
    lens = [r.randint(0, max_len) for _ in range(B)]
    say(f"random paged seed={seed} B={B} H={H} H_kv={H_kv} D={D} bs={bs} lens={lens} {dtype}")
    q, kp, vp, table, kl = workloads.random_paged_case(6000 + seed, B, H, H_kv, D, bs, max_len,
                                                       dtype, lengths=lens)
    ref = oracle.gqa_paged(np64(q), np64(kp), np64(vp), table.numpy(), kl.numpy())
    out = gqa.decode_paged(*(t.cuda() for t in (q, kp, vp, table, kl)))
    torch.cuda.synchronize()
    compare(out, ref, TOL[dtype], f"random paged {seed}")
