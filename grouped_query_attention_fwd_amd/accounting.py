"""Algorithmic byte and flop counts used to express measured times as
bandwidth and throughput (pure host arithmetic, no GPU code).

kv_cache_bytes is the KV-cache equation of the *Theory* section of
"Multi-Query Attention": 2 * L * n * h_kv * d_head * b * sizeof(dtype)
(K and V, L layers, n cached tokens, batch b).
"""

from __future__ import annotations

__all__ = ["kv_cache_bytes", "decode_bytes", "paged_decode_bytes", "visible_pairs",
           "band_pairs", "prefill_flops", "band_flops", "DTYPE_BYTES"]

DTYPE_BYTES = {"fp32": 4, "bf16": 2}


def kv_cache_bytes(L, n, h_kv, d_head, b, sizeof):
    return 2 * L * n * h_kv * d_head * b * sizeof


def decode_bytes(B, H, H_kv, M, D, elt, out_elt=None, include_qo=False):
    """KV bytes one decode call must read (one layer, n = M).  With
    include_qo the query read and output write are added."""
    kv = kv_cache_bytes(1, M, H_kv, D, B, elt)
    if not include_qo:
        return kv
    out_elt = elt if out_elt is None else out_elt
    return kv + B * H * D * elt + B * H * D * out_elt


def paged_decode_bytes(lengths, H_kv, D, elt):
    """KV bytes one paged decode call must read: each sequence's own cached
    keys only (n = kv_len[b], one layer), summed over the batch."""
    return sum(kv_cache_bytes(1, max(0, int(n)), H_kv, D, 1, elt) for n in lengths)


def visible_pairs(N, M, causal=False, lengths=None):
    """Number of visible (query, key) pairs per (batch row, head).

    causal: key j visible to query i iff j <= i; lengths: key j visible iff
    j < length.  Returns a list with one count per batch row when lengths is
    given, else an int."""
    def count(limit):
        if not causal:
            return N * limit
        return sum(min(i + 1, limit) for i in range(N))
    if lengths is None:
        return count(M)
    return [count(min(int(x), M)) for x in lengths]


def prefill_flops(B, H, N, M, D, causal=False, lengths=None):
    """4 * D flop per visible pair (2 for the Q.K dot product, 2 for the
    P.V accumulation), summed over batch rows and heads."""
    vp = visible_pairs(N, M, causal, lengths)
    if lengths is None:
        return 4 * D * H * B * vp
    return 4 * D * H * sum(vp)


def band_pairs(N, M, q_offset=0, window_left=-1, window_right=-1):
    """Visible (query, key) pairs per (batch row, head) for the band
    i + q_offset - window_left <= j <= i + q_offset + window_right
    (negative window = open side), keys in [0, M)."""
    total = 0
    for i in range(N):
        p = i + q_offset
        lo = 0 if window_left < 0 else max(0, p - window_left)
        hi = M - 1 if window_right < 0 else min(M - 1, p + window_right)
        total += max(0, hi - lo + 1)
    return total


def band_flops(B, H, N, M, D, q_offset=0, window_left=-1, window_right=-1):
    """4 * D flop per visible pair of the band, over batch rows and heads."""
    return 4 * D * H * B * band_pairs(N, M, q_offset, window_left, window_right)
