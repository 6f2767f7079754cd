"""GPU parity where one (batch row, KV head) slab of K or V, or a paged
pool, is about 2 GiB: byte offsets past 2^31 must not wrap, and the prefill's
whole-tile copies through a buffer descriptor hand over to the clamped copies
once a slab no longer fits its 32-bit range.

The big tensors are zeros except a seeded random region; only keys in that
region are visible (by band, mask or sequence length), so the oracle runs on
the region alone: keys that are not visible contribute nothing (pinned in the
oracle tests).  Each case allocates about 4.3 GB of device memory."""

import sys

import numpy as np
import pytest
import torch

import grouped_query_attention_fwd_amd as gqa
import oracle
import workloads
from tests.parity import TOL, compare, np64

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# Slabs of M rows of 256 bytes (D = 128, bf16): 8388600 rows stay just below
# 2^31 bytes (descriptor copies reach offsets near 2^31, the ragged last tile
# is clamped); 8392741 rows pass it (every tile takes the clamped copies).
@pytest.mark.parametrize("M", [8388600, 8392741])
def test_band_at_the_end_of_a_2gib_slab(M):
    B, H, H_kv, N, D, W, wl = 1, 4, 1, 64, 128, 4096, 255
    say(f"large band case M={M} B={B} H={H} H_kv={H_kv} N={N} D={D} window={wl + 1}")
    q, kr, vr, _ = workloads.random_case(71, B, H, H_kv, N, W, D, BF16)
    # bottom-right band: query i sits at key M - N + i and sees the 256 keys
    # ending there, all inside the last W rows
    ref = oracle.gqa_band(np64(q), np64(kr), np64(vr), None, W - N, wl, 0)
    k = torch.zeros((B, H_kv, M, D), dtype=BF16, device="cuda")
    v = torch.zeros_like(k)
    k[:, :, M - W:] = kr.cuda()
    v[:, :, M - W:] = vr.cuda()
    out = gqa.prefill_band(q.cuda(), k, v, None, M - N, wl, 0)
    torch.cuda.synchronize()
    compare(out, ref, TOL[BF16], f"large band M={M}")
    del k, v, out
    free()


def test_decode_over_a_2gib_slab_with_mask():
    B, H, H_kv, D, M = 1, 4, 1, 128, 8392741
    head, tail = 100, 3000
    say(f"large decode case M={M} B={B} H={H} H_kv={H_kv} D={D} visible={head}+{tail}")
    q, kr, vr, _ = workloads.random_case(72, B, H, H_kv, 1, head + tail, D, BF16)
    ref = oracle.gqa(np64(q), np64(kr), np64(vr))
    k = torch.zeros((B, H_kv, M, D), dtype=BF16, device="cuda")
    v = torch.zeros_like(k)
    k[:, :, :head] = kr[:, :, :head].cuda()
    v[:, :, :head] = vr[:, :, :head].cuda()
    k[:, :, M - tail:] = kr[:, :, head:].cuda()
    v[:, :, M - tail:] = vr[:, :, head:].cuda()
    mask = torch.zeros((B, 1, M), dtype=torch.bool, device="cuda")
    mask[:, :, :head] = True
    mask[:, :, M - tail:] = True
    out = gqa.decode(q.cuda(), k, v, mask)
    torch.cuda.synchronize()
    compare(out, ref, TOL[BF16], "large decode")
    del k, v, mask, out
    free()


def test_paged_blocks_past_2gib_of_pool():
    H, H_kv, D, bs = 8, 1, 128, 16
    per_block = H_kv * bs * D * 2                      # 4096 bytes
    low = (1 << 31) // per_block                       # first block at byte offset 2^31
    num_blocks = low + 2048
    lengths = [700, 333]
    B = len(lengths)
    say(f"large paged case num_blocks={num_blocks} B={B} H={H} H_kv={H_kv} D={D} "
        f"block_size={bs} lengths={lengths}")
    max_blocks = max((L + bs - 1) // bs for L in lengths)
    rng = np.random.default_rng(73)
    # sequence 0 entirely past 2^31 bytes of the pool, sequence 1 alternating
    # between the start of the pool and past 2^31
    ids0 = low + rng.permutation(1024)[:max_blocks]
    ids1 = np.where(np.arange(max_blocks) % 2 == 0, rng.permutation(1024)[:max_blocks],
                    low + 1024 + rng.permutation(1024)[:max_blocks])
    table = np.stack([ids0, ids1]).astype(np.int32)
    k_pool = torch.zeros((num_blocks, H_kv, bs, D), dtype=BF16, device="cuda")
    v_pool = torch.zeros_like(k_pool)
    q_all, refs = [], []
    for b, L in enumerate(lengths):
        q, kr, vr, _ = workloads.random_case(74 + b, 1, H, H_kv, 1, L, D, BF16)
        q_all.append(q)
        refs.append(oracle.gqa(np64(q), np64(kr), np64(vr)))
        for t in range(0, L, bs):
            blk = int(table[b, t // bs])
            n = min(bs, L - t)
            k_pool[blk, :, :n] = kr[0, :, t:t + n].cuda()
            v_pool[blk, :, :n] = vr[0, :, t:t + n].cuda()
    q = torch.cat(q_all).cuda()
    out = gqa.decode_paged(q, k_pool, v_pool, torch.from_numpy(table).cuda(),
                           torch.tensor(lengths, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    compare(out, np.concatenate(refs), TOL[BF16], "large paged")
    del k_pool, v_pool, out
    free()
