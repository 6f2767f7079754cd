"""Plain fp64 CPU oracle for the grouped-query attention forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in the
repository's entry module and the CPU-baseline leg of the benchmark may import
this module.  The product path (the HIP library and its Python binding) never
imports, calls or falls back to it, and this module imports nothing from the
product path.

What it computes, and where each step comes from:

* "28. Grouped-Query Attention (GQA)", sections *Problem*, *Step-by-Step
  Approach* and *Reference solution*: the group size is read off the shapes
  (query heads divided by KV heads, which must divide exactly), K and V are
  expanded to the query-head count by duplicating each KV head `group` times
  contiguously (repeat-interleave, so query head h reads KV head h // group),
  scores are q . k / sqrt(head_dim), a (batch, seq_q, seq_k) boolean mask is
  broadcast over heads with False meaning "set the score to -inf", a softmax
  runs over the key axis and the weights multiply V.
* "Multi-Query Attention", section *Implementation*: the same interface with
  q [B, H, N, D], k/v [B, H_kv, M, D] and H % H_kv == 0.
* "Grouped-Query Attention Explained Simply", section *Minimal
  implementation*: self-attention with a causal mask.  Causal visibility is
  read as "key j is visible to query i iff j <= i" for any N and M
  (top-left aligned), combined with an explicit mask by logical AND.
* "Grouped-Query Attention vs Multi-Head Attention: Understanding GQA
  Implementation", KV-cache buffers and *Summary*: at decode time each
  sequence attends to the keys it has cached so far, stored per KV head.
  `gather_paged` / `gqa_paged` read such a cache kept in fixed-size blocks
  through a per-sequence block table, with one cached length per sequence:
  the result is plain attention over that sequence's first kv_len keys.

* "28. Grouped-Query Attention (GQA)", *Problem*, names sliding-window
  attention as Mistral's companion to GQA without defining it.
  `band_visibility` / `gqa_band` read it as a band around each query's
  position p = i + q_offset in the key sequence: key j is visible iff
  p - window_left <= j <= p + window_right (a negative window leaves that
  side open).  Causal is the band with right edge 0 and no left limit;
  q_offset = M - N places N queries at the end of the M keys (a prefill
  chunk after a cache).

The page's recipe yields NaN for a query row that sees no key (softmax over an
empty set: -inf minus -inf); the oracle keeps that NaN on purpose.

Everything runs in float64 with numpy; inputs are widened exactly (bf16 and
fp32 values are representable in fp64).  K and V are materialised in their
expanded [B, H, M, D] form per batch row, exactly as the pages describe, with
no blocking, fusion or reordering.  The code is deliberately slow and plain.

Parity status: every function here is pinned by the CPU tests in
tests/test_oracle.py (library cross-check, closed forms, invariants,
brute force and planted-mistake checks); none is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["validate_shapes", "group_size", "expand_kv", "visibility",
           "attention_weights", "gqa", "gather_paged", "gqa_paged",
           "band_visibility", "gqa_band"]


def validate_shapes(q, k, v, mask=None):
    """Shape rules of the *Problem* section of "28. Grouped-Query Attention
    (GQA)" and of the docstring in *Implementation* of "Multi-Query
    Attention": q [B,H,N,D], k and v [B,H_kv,M,D], H a multiple of H_kv,
    optional mask [B,N,M]."""
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B, heads, seq, head_dim]")
    B, H, N, D = q.shape
    Bk, H_kv, M, Dk = k.shape
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if Bk != B or Dk != D:
        raise ValueError("batch and head_dim of q and k/v must agree")
    if H_kv < 1 or H % H_kv != 0:
        raise ValueError("query heads must be an exact multiple of KV heads")
    if mask is not None and tuple(mask.shape) != (B, N, M):
        raise ValueError("mask must be [B, N, M]")
    return B, H, H_kv, N, M, D


def group_size(H, H_kv):
    """Group size from the shapes alone (*Step-by-Step Approach*, step 1)."""
    return H // H_kv


def expand_kv(x, group):
    """Repeat-interleave along the head axis (*Step-by-Step Approach*,
    step 2): each KV head is duplicated `group` times contiguously, so the
    expanded head h holds KV head h // group.  This is np.repeat, not np.tile
    (the *Key Functions & Tricks* section warns against tiling)."""
    return np.repeat(x, group, axis=1)


def visibility(B, N, M, mask=None, causal=False):
    """Boolean [B, N, M]: True where query i may attend to key j.

    mask: True = attend (the reference solution fills ~mask with -inf).
    causal: key j visible to query i iff j <= i (self-attention causal mask of
    "Grouped-Query Attention Explained Simply", read top-left aligned).
    Both together combine by AND."""
    vis = np.ones((B, N, M), dtype=bool)
    if mask is not None:
        vis &= np.asarray(mask, dtype=bool)
    if causal:
        i = np.arange(N)[:, None]
        j = np.arange(M)[None, :]
        vis &= (j <= i)[None, :, :]
    return vis


def attention_weights(q, k, mask=None, causal=False):
    """Softmax weights [B, H, N, M] in float64 (*Step-by-Step Approach*,
    steps 3-4; *Reference solution*).  Rows with no visible key are NaN."""
    B, H, H_kv, N, M, D = validate_shapes(q, k, k, mask)
    g = group_size(H, H_kv)
    vis = visibility(B, N, M, mask, causal)
    out = np.empty((B, H, N, M), dtype=np.float64)
    for b in range(B):
        qb = np.asarray(q[b], dtype=np.float64)                  # [H, N, D]
        kb = expand_kv(np.asarray(k[b:b + 1], dtype=np.float64), g)[0]  # [H, M, D]
        scores = np.matmul(qb, kb.transpose(0, 2, 1)) / math.sqrt(D)   # [H, N, M]
        scores = np.where(vis[b][None, :, :], scores, -np.inf)
        with np.errstate(invalid="ignore"):
            row_max = scores.max(axis=-1, keepdims=True)
            e = np.exp(scores - row_max)
            out[b] = e / e.sum(axis=-1, keepdims=True)
    return out


def gqa(q, k, v, mask=None, causal=False):
    """O = softmax(Q K^T / sqrt(D) [masked]) V with repeat-interleave head
    grouping; returns float64 [B, H, N, D].  Runs per batch row to bound
    memory; the expanded K and V of that row are materialised."""
    B, H, H_kv, N, M, D = validate_shapes(q, k, v, mask)
    g = group_size(H, H_kv)
    out = np.empty((B, H, N, D), dtype=np.float64)
    for b in range(B):
        w = attention_weights(q[b:b + 1], k[b:b + 1],
                              None if mask is None else mask[b:b + 1], causal)[0]
        vb = expand_kv(np.asarray(v[b:b + 1], dtype=np.float64), g)[0]  # [H, M, D]
        out[b] = np.matmul(w, vb)
    return out


def gather_paged(k_pool, v_pool, block_table, kv_len):
    """Rebuild the contiguous per-sequence cache from a block pool.

    k_pool, v_pool: [num_blocks, H_kv, block_size, D]; block_table
    [B, max_blocks] of block ids; kv_len [B].  Key t of sequence b and KV
    head j is k_pool[block_table[b, t // block_size], j, t % block_size].
    Returns k, v [B, H_kv, max_blocks * block_size, D] (float64, zero past
    the sequence's length) and the decode mask [B, 1, M] with
    mask[b, 0, t] = t < kv_len[b] (lengths clamped to [0, M])."""
    k_pool = np.asarray(k_pool, dtype=np.float64)
    v_pool = np.asarray(v_pool, dtype=np.float64)
    table = np.asarray(block_table, dtype=np.int64)
    lens = np.asarray(kv_len, dtype=np.int64)
    num_blocks, H_kv, bs, D = k_pool.shape
    B, max_blocks = table.shape
    M = max_blocks * bs
    k = np.zeros((B, H_kv, M, D))
    v = np.zeros((B, H_kv, M, D))
    mask = np.zeros((B, 1, M), dtype=bool)
    for b in range(B):
        n = min(max(int(lens[b]), 0), M)
        for t in range(n):
            blk = int(table[b, t // bs])
            if not 0 <= blk < num_blocks:
                raise ValueError("block id outside the pool")
            k[b, :, t, :] = k_pool[blk, :, t % bs, :]
            v[b, :, t, :] = v_pool[blk, :, t % bs, :]
            mask[b, 0, t] = True
    return k, v, mask


def gqa_paged(q, k_pool, v_pool, block_table, kv_len):
    """Decode (q [B, H, 1, D]) over a paged cache: gqa() on the gathered
    cache with the length mask."""
    k, v, mask = gather_paged(k_pool, v_pool, block_table, kv_len)
    return gqa(q, k, v, mask)


def band_visibility(N, M, q_offset=0, window_left=-1, window_right=-1):
    """Boolean [N, M]: key j visible to query i iff
    (window_left < 0 or j >= i + q_offset - window_left) and
    (window_right < 0 or j <= i + q_offset + window_right)."""
    i = np.arange(N)[:, None]
    j = np.arange(M)[None, :]
    pos = i + q_offset
    vis = np.ones((N, M), dtype=bool)
    if window_left >= 0:
        vis &= j >= pos - window_left
    if window_right >= 0:
        vis &= j <= pos + window_right
    return vis


def gqa_band(q, k, v, mask=None, q_offset=0, window_left=-1, window_right=-1):
    """gqa() with the band of band_visibility ANDed into the mask (the band
    is the same for every batch row and head)."""
    B, H, H_kv, N, M, D = validate_shapes(q, k, v, mask)
    vis = np.broadcast_to(band_visibility(N, M, q_offset, window_left, window_right),
                          (B, N, M))
    if mask is not None:
        vis = vis & np.asarray(mask, dtype=bool)
    return gqa(q, k, v, np.ascontiguousarray(vis))
