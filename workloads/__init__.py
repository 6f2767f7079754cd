"""Seeded synthetic inputs for the grouped-query attention forward pass.

This module holds the five workload definitions and the random-input
generators that feed both the HIP path and the fp64 oracle.  It contains none
of the attention arithmetic: it only draws numbers and builds the padding mask
that defines a workload.

Recipe (same bits for both sides):
  * a CPU ``torch.Generator`` seeded with the workload's seed;
  * draw q, then k, then v as float32 N(0, 1) in that order;
  * cast to bfloat16 or float16 for 16-bit workloads (round-to-nearest-even);
  * padded workloads then draw one length per batch row, uniform on
    {1, ..., M}, and key j is valid for batch row b iff j < len_b.

Shapes follow the pages: Mistral-7B heads (32 query / 8 KV) and Llama-2-70B
heads (64 / 8) from "Grouped-Query Attention Explained Simply", *Numbers to
anchor on*; 4K and 32k contexts and batch 16 from the KV-cache figures of the
GQA deep-dive page and of "Multi-Query Attention"; the (4, 512, d_model=768,
32 heads, 4 KV heads) usage example of the deep-dive page's *Implementation*
section gives head_dim 24 for the padded workload; the tiny workload is the
worked example of "28. Grouped-Query Attention (GQA)", *Problem*.
"""

from __future__ import annotations

import dataclasses

import torch

__all__ = ["Workload", "WORKLOADS", "GROUP_SWEEP", "by_name", "make_inputs", "random_case",
           "PagedWorkload", "PAGED_WORKLOADS", "paged_by_name", "make_paged_inputs",
           "random_paged_case", "KEY_PATTERN_MOD", "KEY_PATTERN_POISON", "key_pattern_rows",
           "key_coverage_inputs", "key_coverage_paged"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    H: int
    H_kv: int
    N: int
    M: int
    D: int
    dtype: str          # "fp32" or "bf16"
    causal: bool = False
    padded: bool = False  # padding mask j < len_b, len_b ~ U{1..M}
    # band around position i + q_offset: window_left keys before, window_right
    # after (-1 = open); used by the banded prefill workloads
    q_offset: int = 0
    window_left: int = -1
    window_right: int = -1

    @property
    def band(self):
        if self.q_offset == 0 and self.window_left < 0 and self.window_right < 0:
            return None
        return (self.q_offset, self.window_left, self.window_right)

    @property
    def kind(self) -> str:
        return "decode" if self.N == 1 and not self.causal and self.band is None else "prefill"

    @property
    def torch_dtype(self):
        return {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[self.dtype]


WORKLOADS = [
    Workload("tiny_fp32", 1, 1, 4, 2, 5, 5, 4, "fp32"),
    Workload("decode_mistral7b_m4096", 2, 16, 32, 8, 1, 4096, 128, "bf16"),
    Workload("decode_llama70b_m32768", 3, 16, 64, 8, 1, 32768, 128, "bf16"),
    Workload("prefill_causal_n4096", 4, 4, 32, 8, 4096, 4096, 128, "bf16",
             causal=True),
    Workload("prefill_padded_d24", 5, 4, 32, 4, 512, 512, 24, "fp32",
             padded=True),
    # sliding window of 4096 keys (Mistral-style local attention) over a
    # 16K-token self-attention prefill
    Workload("prefill_window4096_n16384", 8, 1, 32, 8, 16384, 16384, 128, "bf16",
             window_left=4095, window_right=0),
    # a 512-token prefill chunk appended to 3584 cached keys: bottom-right
    # causal over M = 4096
    Workload("prefill_chunk512_m4096", 9, 16, 32, 8, 512, 4096, 128, "bf16",
             q_offset=3584, window_right=0),
    # the headline decode and causal prefill shapes with fp16 inputs
    Workload("decode_mistral7b_m4096_fp16", 10, 16, 32, 8, 1, 4096, 128, "fp16"),
    Workload("prefill_causal_n4096_fp16", 11, 4, 32, 8, 4096, 4096, 128, "fp16",
             causal=True),
    # causal prefill with 256-wide heads (the kernel's largest head size)
    Workload("prefill_causal_n4096_d256", 12, 2, 16, 4, 4096, 4096, 256, "bf16",
             causal=True),
]


# Group-size sweep: decode with 64 query heads and g = H / H_kv from 1 (MHA,
# 64 KV heads) to 64 (MQA, one KV head), B16, M 4096, D 128, bf16.
GROUP_SWEEP = [
    Workload(f"decode_h64_g{g}_m4096", 100 + g, 16, 64, 64 // g, 1, 4096, 128, "bf16")
    for g in (1, 2, 4, 8, 16, 32, 64)
]


def by_name(name: str) -> Workload:
    for w in WORKLOADS + GROUP_SWEEP:
        if w.name == name:
            return w
    raise KeyError(name)


def _draw(gen, B, H, H_kv, N, M, D, dtype):
    q = torch.randn((B, H, N, D), generator=gen, dtype=torch.float32)
    k = torch.randn((B, H_kv, M, D), generator=gen, dtype=torch.float32)
    v = torch.randn((B, H_kv, M, D), generator=gen, dtype=torch.float32)
    if dtype in (torch.bfloat16, torch.float16):
        q, k, v = q.to(dtype), k.to(dtype), v.to(dtype)
    return q, k, v


def padding_mask(lengths, N, M):
    """mask[b, i, j] = j < lengths[b] (True = key valid), shape [B, N, M]."""
    j = torch.arange(M)
    row = j[None, :] < lengths[:, None]                     # [B, M]
    return row[:, None, :].expand(len(lengths), N, M).contiguous()


def make_inputs(w: Workload):
    """Return (q, k, v, mask, causal) as CPU tensors for workload ``w``.

    mask is a bool tensor [B, N, M] or None."""
    gen = torch.Generator().manual_seed(w.seed)
    q, k, v = _draw(gen, w.B, w.H, w.H_kv, w.N, w.M, w.D, w.torch_dtype)
    mask = None
    if w.padded:
        lengths = torch.randint(1, w.M + 1, (w.B,), generator=gen)
        mask = padding_mask(lengths, w.N, w.M)
    return q, k, v, mask, w.causal


def random_case(seed, B, H, H_kv, N, M, D, dtype=torch.float32,
                mask_kind=None, q_scale=1.0):
    """Small randomized case for parity sweeps.

    mask_kind: None, "padding" (j < len_b), "random" (i.i.d. Bernoulli(0.7)
    per [b, i, j]) or "blocks" (whole 64-key column blocks switched off at
    random, to exercise skipped tiles).  q_scale multiplies q before the
    cast, to make peaky score rows."""
    gen = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, N, D), generator=gen, dtype=torch.float32) * q_scale
    k = torch.randn((B, H_kv, M, D), generator=gen, dtype=torch.float32)
    v = torch.randn((B, H_kv, M, D), generator=gen, dtype=torch.float32)
    if dtype in (torch.bfloat16, torch.float16):
        q, k, v = q.to(dtype), k.to(dtype), v.to(dtype)
    mask = None
    if mask_kind == "padding":
        lengths = torch.randint(1, M + 1, (B,), generator=gen)
        mask = padding_mask(lengths, N, M)
    elif mask_kind == "random":
        mask = torch.rand((B, N, M), generator=gen) < 0.7
    elif mask_kind == "blocks":
        nblk = (M + 63) // 64
        on = torch.rand((B, nblk), generator=gen) < 0.5
        on[:, 0] = True
        cols = on.repeat_interleave(64, dim=1)[:, :M]        # [B, M]
        mask = cols[:, None, :].expand(B, N, M).contiguous()
    elif mask_kind is not None:
        raise ValueError(mask_kind)
    return q, k, v, mask


# ------------------------------------------------------------ paged KV cache
@dataclasses.dataclass(frozen=True)
class PagedWorkload:
    """Decode over a KV cache kept in blocks of ``block_size`` keys.

    Each of the B sequences has its own cached length; ``lengths`` is
    "full" (every sequence holds max_len keys) or "uniform" (length drawn
    uniformly from {1, ..., max_len}).  Blocks are scattered over the pool
    in a random order."""
    name: str
    seed: int
    B: int
    H: int
    H_kv: int
    max_len: int
    D: int
    block_size: int
    dtype: str
    lengths: str = "uniform"

    @property
    def max_blocks(self) -> int:
        return -(-self.max_len // self.block_size)

    @property
    def torch_dtype(self):
        return {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[self.dtype]


PAGED_WORKLOADS = [
    # the Mistral-7B-shaped decode batch with serving-style mixed lengths
    PagedWorkload("decode_paged_mistral7b_varlen", 6, 16, 32, 8, 4096, 128, 16, "bf16"),
    # the same batch with every sequence full: same bytes as the contiguous decode
    PagedWorkload("decode_paged_mistral7b_full", 7, 16, 32, 8, 4096, 128, 16, "bf16",
                  lengths="full"),
]


def paged_by_name(name: str) -> PagedWorkload:
    for w in PAGED_WORKLOADS:
        if w.name == name:
            return w
    raise KeyError(name)


def random_paged_case(seed, B, H, H_kv, D, block_size, max_len, dtype=torch.float32,
                      lengths="uniform", slack_blocks=3, shared_first_block=False,
                      q_scale=1.0):
    """(q, k_pool, v_pool, block_table, kv_len) as CPU tensors.

    Draw order: q [B,H,1,D], then the pool K and V [num_blocks, H_kv,
    block_size, D] as float32 N(0,1) (cast afterwards for bf16), then the
    lengths, then a random permutation that scatters the blocks.  lengths:
    "uniform" (U{1..max_len}), "full", or an explicit list (0 allowed).
    Table entries past a sequence's last block are -1 (never read).
    shared_first_block: sequence 1 reuses sequence 0's first block (a shared
    prefix), which is legal."""
    gen = torch.Generator().manual_seed(seed)
    max_blocks = -(-max_len // block_size)
    if isinstance(lengths, str):
        probe = torch.Generator().manual_seed(seed + 1_000_003)
        if lengths == "full":
            lens = torch.full((B,), max_len, dtype=torch.int64)
        elif lengths == "uniform":
            lens = torch.randint(1, max_len + 1, (B,), generator=probe)
        else:
            raise ValueError(lengths)
    else:
        lens = torch.tensor(list(lengths), dtype=torch.int64)
    need = [-(-int(n) // block_size) for n in lens]
    num_blocks = sum(need) + slack_blocks
    q = torch.randn((B, H, 1, D), generator=gen, dtype=torch.float32) * q_scale
    kp = torch.randn((num_blocks, H_kv, block_size, D), generator=gen, dtype=torch.float32)
    vp = torch.randn((num_blocks, H_kv, block_size, D), generator=gen, dtype=torch.float32)
    if dtype in (torch.bfloat16, torch.float16):
        q, kp, vp = q.to(dtype), kp.to(dtype), vp.to(dtype)
    perm = torch.randperm(num_blocks, generator=gen)
    table = torch.full((B, max_blocks), -1, dtype=torch.int32)
    at = 0
    for b in range(B):
        table[b, :need[b]] = perm[at:at + need[b]].to(torch.int32)
        at += need[b]
    if shared_first_block and B > 1 and need[0] > 0 and need[1] > 0:
        table[1, 0] = table[0, 0]
    return q, kp, vp, table, lens.to(torch.int32)


def make_paged_inputs(w: PagedWorkload):
    return random_paged_case(w.seed, w.B, w.H, w.H_kv, w.D, w.block_size, w.max_len,
                             w.torch_dtype, lengths=w.lengths, slack_blocks=0)


# ------------------------------------------------- key-coverage check inputs
# V holds small integers that vary with the key index without a short
# period, and K is zero, so every visible key gets the same weight and the
# attention output is the plain mean of V over the visible keys: a closed
# form that sees a skipped, repeated or shifted key.  All values are exact
# in bf16, fp16 and fp32, and sums over up to 67,000 keys stay below 2^24,
# so every partial sum in fp32 is exact too.
KEY_PATTERN_MOD = 251        # a prime, so no power-of-two key range is a whole period
KEY_PATTERN_POISON = 255     # for pool rows that no sequence owns (exact in 16 bits)


def key_pattern_rows(b, H_kv, m0, m1, D):
    """int32 [H_kv, m1 - m0, D]: V[b, j, m, d] = (7 m + 13 d + 29 j + 31 b) mod 251
    for keys m0 <= m < m1."""
    j = torch.arange(H_kv, dtype=torch.int64)[:, None, None]
    m = torch.arange(m0, m1, dtype=torch.int64)[None, :, None]
    d = torch.arange(D, dtype=torch.int64)[None, None, :]
    return ((7 * m + 13 * d + 29 * j + 31 * b) % KEY_PATTERN_MOD).to(torch.int32)


def key_coverage_inputs(B, H, H_kv, N, M, D, dtype):
    """(q, k, v) CPU tensors for a key-coverage check: q i.i.d. N(0,1) (its
    values do not matter, K is zero), k = 0, v = key_pattern_rows."""
    gen = torch.Generator().manual_seed(7919)
    q = torch.randn((B, H, N, D), generator=gen, dtype=torch.float32).to(dtype)
    k = torch.zeros((B, H_kv, M, D), dtype=dtype)
    v = torch.empty((B, H_kv, M, D), dtype=dtype)
    for b in range(B):
        v[b] = key_pattern_rows(b, H_kv, 0, M, D).to(dtype)
    return q, k, v


def key_coverage_paged(w: PagedWorkload):
    """(q, k_pool, v_pool, block_table, kv_len) for a key-coverage check of a
    paged workload: its block table and lengths, K zero, and the pool V
    filled so that key t of sequence b holds key_pattern_rows(b, ...)[:, t];
    pool rows owned by no sequence hold KEY_PATTERN_POISON."""
    q, kp, vp, table, lens = make_paged_inputs(w)
    dtype = w.torch_dtype
    kp = torch.zeros_like(kp)
    vp = torch.full(vp.shape, KEY_PATTERN_POISON, dtype=dtype)
    bs = w.block_size
    for b in range(w.B):
        n = int(lens[b])
        rows = key_pattern_rows(b, w.H_kv, 0, n, w.D).to(dtype)      # [H_kv, n, D]
        for t0 in range(0, n, bs):
            blk = int(table[b, t0 // bs])
            t1 = min(n, t0 + bs)
            vp[blk, :, : t1 - t0, :] = rows[:, t0:t1, :]
    return q, kp, vp, table, lens
