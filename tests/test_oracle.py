"""Pins for the fp64 oracle: it is checked against things other than itself.

* a library routine that computes the same thing (torch's CPU
  scaled_dot_product_attention with enable_gqa, float64);
* closed forms (single key, two keys, all-zero keys, constant-per-head V);
* invariants (weights sum to one, masked keys contribute nothing, padding
  equals truncation, causal equals an explicit lower-triangular mask, key
  permutation);
* pure-Python brute force on tiny inputs;
* the worked example of "28. Grouped-Query Attention (GQA)" (shape only);
* planted mistakes: mutated copies of the oracle must fail at least one pin.
"""

import math
import os
import re
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import gqa_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


def rand_qkv(seed, B, H, H_kv, N, M, D, scale=1.0):
    r = rng(seed)
    q = r.standard_normal((B, H, N, D)) * scale
    k = r.standard_normal((B, H_kv, M, D))
    v = r.standard_normal((B, H_kv, M, D))
    return q, k, v


def brute_force(q, k, v, mask=None, causal=False):
    """Pure-Python loops (math.exp, explicit sums) over tiny inputs."""
    B, H, N, D = q.shape
    H_kv, M = k.shape[1], k.shape[2]
    g = H // H_kv
    out = np.zeros((B, H, N, D))
    for b in range(B):
        for h in range(H):
            j = h // g
            for i in range(N):
                s = []
                for m in range(M):
                    ok = True
                    if mask is not None and not mask[b][i][m]:
                        ok = False
                    if causal and m > i:
                        ok = False
                    if ok:
                        dot = 0.0
                        for d in range(D):
                            dot += float(q[b, h, i, d]) * float(k[b, j, m, d])
                        s.append((m, dot / math.sqrt(D)))
                if not s:
                    out[b, h, i, :] = float("nan")
                    continue
                mx = max(x for _, x in s)
                w = [(m, math.exp(x - mx)) for m, x in s]
                tot = sum(x for _, x in w)
                for d in range(D):
                    out[b, h, i, d] = sum(x * float(v[b, j, m, d]) for m, x in w) / tot
    return out


def rand_paged(seed, B, H, H_kv, D, bs, lens, max_blocks, slack=3):
    """Random pool, a random block assignment (blocks shuffled over the pool,
    unused table entries -1) and the given lengths."""
    r = rng(seed)
    need = [-(-min(n, max_blocks * bs) // bs) for n in lens]
    nb = sum(need) + slack
    q = r.standard_normal((B, H, 1, D))
    kp = r.standard_normal((nb, H_kv, bs, D))
    vp = r.standard_normal((nb, H_kv, bs, D))
    perm = r.permutation(nb)
    table = -np.ones((B, max_blocks), dtype=np.int64)
    at = 0
    for b in range(B):
        table[b, :need[b]] = perm[at:at + need[b]]
        at += need[b]
    return q, kp, vp, table, np.asarray(lens)


def brute_force_paged(q, kp, vp, table, lens):
    """Pure-Python decode over a paged cache, indexing the pool per key."""
    B, H, _, D = q.shape
    H_kv, bs = kp.shape[1], kp.shape[2]
    g = H // H_kv
    out = np.zeros((B, H, 1, D))
    for b in range(B):
        for h in range(H):
            j = h // g
            s = []
            for t in range(int(lens[b])):
                blk, off = int(table[b][t // bs]), t % bs
                dot = sum(float(q[b, h, 0, d]) * float(kp[blk, j, off, d]) for d in range(D))
                s.append(((blk, off), dot / math.sqrt(D)))
            if not s:
                out[b, h, 0, :] = float("nan")
                continue
            mx = max(x for _, x in s)
            w = [(loc, math.exp(x - mx)) for loc, x in s]
            tot = sum(x for _, x in w)
            for d in range(D):
                out[b, h, 0, d] = sum(x * float(vp[blk, j, off, d])
                                      for (blk, off), x in w) / tot
    return out


# ---------------------------------------------------------------- pin suite
# Each pin takes an oracle module and raises AssertionError (or any error)
# when the module disagrees with what the pages and the mathematics fix.

def pin_worked_example_shape(orc):
    shapes = {}
    with open(os.path.join(GOLDEN, "worked_example.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, *dims = line.split()
                shapes[name] = tuple(int(x) for x in dims)
    r = rng(0)
    q = r.standard_normal(shapes["q"])
    k = r.standard_normal(shapes["k"])
    assert orc.gqa(q, k, k).shape == shapes["out"]


def _sdpa_ref(q, k, v, mask=None, causal=False):
    """torch CPU SDPA in float64, grouping via enable_gqa."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    N, M = q.shape[2], k.shape[2]
    attn = None
    if mask is not None:
        attn = torch.from_numpy(mask)[:, None, :, :]
    if causal:
        tri = torch.ones(N, M, dtype=torch.bool).tril()
        attn = tri[None, None] if attn is None else (attn & tri[None, None])
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=attn,
                                       enable_gqa=(q.shape[1] != k.shape[1]))
    return o.numpy()


LIB_CASES = [
    # seed, B, H, H_kv, N, M, D, mask kind, causal
    (1, 2, 4, 4, 7, 9, 8, None, False),     # MHA
    (2, 2, 8, 2, 5, 13, 16, None, False),   # g = 4
    (3, 1, 6, 3, 6, 6, 4, None, True),      # g = 2, causal N == M
    (4, 2, 4, 1, 3, 11, 8, "random", False),  # MQA with mask
    (5, 2, 8, 4, 9, 5, 12, "padding", False),
    (6, 1, 4, 2, 8, 12, 8, "random", True),  # mask AND causal, N != M
]


def _mask(kind, seed, B, N, M):
    r = rng(seed + 1000)
    if kind is None:
        return None
    if kind == "random":
        m = r.random((B, N, M)) < 0.6
        m[:, :, 0] = True          # every row sees key 0 (SDPA differs on empty rows)
        return m
    lens = r.integers(1, M + 1, size=B)
    return np.broadcast_to(np.arange(M)[None, None, :] < lens[:, None, None],
                           (B, N, M)).copy()


def pin_library_crosscheck(orc):
    for seed, B, H, H_kv, N, M, D, mk, causal in LIB_CASES:
        q, k, v = rand_qkv(seed, B, H, H_kv, N, M, D)
        mask = _mask(mk, seed, B, N, M)
        ref = _sdpa_ref(q, k, v, mask, causal)
        got = orc.gqa(q, k, v, mask, causal)
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def pin_brute_force(orc):
    cases = [(11, 1, 4, 2, 3, 5, 3, None, False),
             (12, 2, 2, 1, 4, 4, 2, "random", True),
             (13, 1, 6, 2, 2, 7, 4, "padding", False),
             (14, 1, 3, 3, 3, 3, 5, None, True)]
    for seed, B, H, H_kv, N, M, D, mk, causal in cases:
        q, k, v = rand_qkv(seed, B, H, H_kv, N, M, D)
        mask = _mask(mk, seed, B, N, M)
        np.testing.assert_allclose(orc.gqa(q, k, v, mask, causal),
                                   brute_force(q, k, v, mask, causal),
                                   rtol=1e-12, atol=1e-13)


def pin_mha_equals_per_head(orc):
    """H_kv == H is ordinary multi-head attention ("Step-by-Step Approach",
    sanity check): compared with torch SDPA without grouping and with the
    brute-force loops."""
    q, k, v = rand_qkv(21, 2, 3, 3, 4, 6, 5)
    got = orc.gqa(q, k, v)
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(x) for x in (q, k, v))).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got, brute_force(q, k, v), rtol=1e-12, atol=1e-13)


def pin_mqa_brute_force(orc):
    """H_kv == 1: every query head reads the single KV head."""
    q, k, v = rand_qkv(22, 1, 5, 1, 3, 6, 4)
    got = orc.gqa(q, k, v)
    for h in range(5):
        one = brute_force(q[:, h:h + 1], k, v)
        np.testing.assert_allclose(got[:, h:h + 1], one, rtol=1e-12, atol=1e-13)


def pin_single_key(orc):
    """M == 1: the softmax weight is exactly 1, so out[b,h] = v[b, h//g, 0]."""
    q, k, v = rand_qkv(23, 2, 8, 2, 3, 1, 6)
    got = orc.gqa(q, k, v)
    for h in range(8):
        assert np.array_equal(got[:, h], np.broadcast_to(v[:, h // 4, 0:1, :], (2, 3, 6)))


def pin_two_keys_closed_form(orc):
    """M == 2: weight of key 1 is the logistic of (s1 - s0) with
    s = q.k / sqrt(D)."""
    q, k, v = rand_qkv(24, 1, 4, 2, 3, 2, 9)
    got = orc.gqa(q, k, v)
    for h in range(4):
        j = h // 2
        for i in range(3):
            s0 = float(np.dot(q[0, h, i], k[0, j, 0])) / 3.0
            s1 = float(np.dot(q[0, h, i], k[0, j, 1])) / 3.0
            w1 = 1.0 / (1.0 + math.exp(s0 - s1))
            ref = (1.0 - w1) * v[0, j, 0] + w1 * v[0, j, 1]
            np.testing.assert_allclose(got[0, h, i], ref, rtol=1e-12, atol=1e-13)


def pin_scale_exact(orc):
    """Scores carry exactly 1/sqrt(D): with D = 4, q = (2,0,0,0), k0 = e0 and
    k1 = 0 the scores are 1 and 0, so the weights are e/(e+1) and 1/(e+1)."""
    q = np.zeros((1, 1, 1, 4)); q[0, 0, 0, 0] = 2.0
    k = np.zeros((1, 1, 2, 4)); k[0, 0, 0, 0] = 1.0
    v = np.zeros((1, 1, 2, 4)); v[0, 0, 0, :] = 1.0
    got = orc.gqa(q, k, v)
    e = math.e
    np.testing.assert_allclose(got[0, 0, 0], np.full(4, e / (e + 1)), rtol=1e-14)


def pin_zero_keys_give_mean(orc):
    """K == 0 makes all visible scores equal, so the output is the mean of
    the visible V rows of the head's KV head (mask and causal included)."""
    B, H, H_kv, N, M, D = 2, 6, 2, 5, 7, 3
    q, _, v = rand_qkv(25, B, H, H_kv, N, M, D)
    k = np.zeros((B, H_kv, M, D))
    mask = _mask("random", 25, B, N, M)
    got = orc.gqa(q, k, v, mask, causal=True)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                vis = [m for m in range(M) if mask[b, i, m] and m <= i]
                ref = v[b, h // 3, vis].mean(axis=0)
                np.testing.assert_allclose(got[b, h, i], ref, rtol=1e-12, atol=1e-14)


def pin_head_mapping_exact(orc):
    """K == 0 and V[b, j] == j: query head h must return exactly h // g
    (repeat-interleave); the tiled mapping h % H_kv would differ.  M is a
    power of two so that the equal weights 1/M are exact in binary."""
    for H, H_kv in [(8, 2), (12, 4), (6, 3), (4, 4), (5, 1)]:
        g = H // H_kv
        q = rng(26).standard_normal((2, H, 3, 4))
        k = np.zeros((2, H_kv, 8, 4))
        v = np.broadcast_to(np.arange(H_kv, dtype=np.float64)[None, :, None, None],
                            (2, H_kv, 8, 4)).copy()
        got = orc.gqa(q, k, v)
        for h in range(H):
            assert np.all(got[:, h] == h // g), (H, H_kv, h)


def pin_weights_sum_to_one(orc):
    q, k, _ = rand_qkv(27, 2, 8, 4, 6, 10, 8, scale=3.0)
    mask = _mask("random", 27, 2, 6, 10)
    w = orc.attention_weights(q, k, mask, causal=True)
    np.testing.assert_allclose(w.sum(axis=-1), 1.0, rtol=0, atol=1e-14)
    assert np.all(w >= 0)
    # masked or future keys get exactly zero weight
    vis = mask[:, None] & (np.arange(10)[None, :] <= np.arange(6)[:, None])[None, None]
    assert np.all(w[~np.broadcast_to(vis, w.shape)] == 0.0)


def pin_masked_keys_contribute_nothing(orc):
    B, H, H_kv, N, M, D = 2, 4, 2, 5, 9, 6
    q, k, v = rand_qkv(28, B, H, H_kv, N, M, D)
    lens = np.array([4, 7])
    mask = np.arange(M)[None, None, :] < lens[:, None, None]
    mask = np.broadcast_to(mask, (B, N, M)).copy()
    a = orc.gqa(q, k, v, mask)
    k2, v2 = k.copy(), v.copy()
    for b in range(B):
        k2[b, :, lens[b]:] = 1e3 * rng(29).standard_normal(k2[b, :, lens[b]:].shape)
        v2[b, :, lens[b]:] = -7.0
    assert np.array_equal(a, orc.gqa(q, k2, v2, mask))
    # padding mask equals attention over the truncated key set
    for b in range(B):
        t = orc.gqa(q[b:b + 1], k[b:b + 1, :, :lens[b]], v[b:b + 1, :, :lens[b]])
        np.testing.assert_allclose(a[b:b + 1], t, rtol=1e-13, atol=1e-14)


def pin_causal_properties(orc):
    B, H, H_kv, N, D = 2, 4, 2, 6, 5
    q, k, v = rand_qkv(30, B, H, H_kv, N, N, D)
    c = orc.gqa(q, k, v, causal=True)
    tri = np.broadcast_to(np.tril(np.ones((N, N), dtype=bool)), (B, N, N)).copy()
    np.testing.assert_allclose(c, orc.gqa(q, k, v, tri), rtol=1e-14, atol=1e-15)
    full = orc.gqa(q, k, v)
    np.testing.assert_allclose(c[:, :, -1], full[:, :, -1], rtol=1e-13, atol=1e-14)
    for h in range(H):
        assert np.array_equal(c[:, h, 0], v[:, h // 2, 0])
    # N != M: causal is top-left (key j visible to query i iff j <= i)
    q2, k2, v2 = rand_qkv(31, 1, 2, 1, 3, 7, 4)
    c2 = orc.gqa(q2, k2, v2, causal=True)
    for i in range(3):
        sub = orc.gqa(q2[:, :, i:i + 1], k2[:, :, :i + 1], v2[:, :, :i + 1])
        np.testing.assert_allclose(c2[:, :, i:i + 1], sub, rtol=1e-13, atol=1e-14)


def pin_key_permutation(orc):
    B, H, H_kv, N, M, D = 1, 4, 2, 3, 8, 4
    q, k, v = rand_qkv(32, B, H, H_kv, N, M, D)
    mask = _mask("random", 32, B, N, M)
    perm = rng(33).permutation(M)
    a = orc.gqa(q, k, v, mask)
    b = orc.gqa(q, k[:, :, perm], v[:, :, perm], mask[:, :, perm])
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


def pin_empty_row_is_nan(orc):
    """A row with no visible key follows the reference solution's recipe
    (softmax of all -inf), i.e. NaN; rows that see keys stay finite."""
    q, k, v = rand_qkv(34, 1, 4, 2, 3, 4, 4)
    mask = np.ones((1, 3, 4), dtype=bool)
    mask[0, 1, :] = False
    o = orc.gqa(q, k, v, mask)
    assert np.all(np.isnan(o[0, :, 1]))
    assert np.all(np.isfinite(o[0, :, 0])) and np.all(np.isfinite(o[0, :, 2]))


def pin_rejects_bad_group(orc):
    q, k, v = rand_qkv(35, 1, 6, 4, 2, 3, 4)
    with pytest.raises(ValueError):
        orc.gqa(q, k, v)


def pin_paged_brute_force(orc):
    """Paged decode equals per-key brute force over the pool (empty
    sequence -> NaN, lengths ending mid-block, block ids shuffled)."""
    q, kp, vp, table, lens = rand_paged(60, 4, 6, 2, 4, 3, [7, 0, 9, 1], max_blocks=4)
    got = orc.gqa_paged(q, kp, vp, table, lens)
    ref = brute_force_paged(q, kp, vp, table, lens)
    assert np.isnan(got[1]).all()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def pin_paged_identity_table(orc):
    """A contiguous cache cut into blocks in order, with full lengths, is
    the unpaged decode exactly."""
    B, H, H_kv, M, D, bs = 2, 8, 2, 12, 4, 4
    q, k, v = rand_qkv(61, B, H, H_kv, 1, M, D)
    mb = M // bs
    # [B, H_kv, mb, bs, D] -> [B, mb, H_kv, bs, D] -> pool [B*mb, H_kv, bs, D]
    kp = k.reshape(B, H_kv, mb, bs, D).transpose(0, 2, 1, 3, 4).reshape(B * mb, H_kv, bs, D)
    vp = v.reshape(B, H_kv, mb, bs, D).transpose(0, 2, 1, 3, 4).reshape(B * mb, H_kv, bs, D)
    table = np.arange(B * mb).reshape(B, mb)
    got = orc.gqa_paged(q, kp, vp, table, np.full(B, M))
    assert np.array_equal(got, orc.gqa(q, k, v))


def pin_paged_length_is_truncation(orc):
    """Only the first kv_len keys count: equal to the unpaged decode of the
    truncated cache, for lengths inside and at the end of blocks."""
    B, H, H_kv, M, D, bs = 3, 4, 2, 16, 4, 4
    q, k, v = rand_qkv(62, B, H, H_kv, 1, M, D)
    mb = M // bs
    kp = k.reshape(B, H_kv, mb, bs, D).transpose(0, 2, 1, 3, 4).reshape(B * mb, H_kv, bs, D)
    vp = v.reshape(B, H_kv, mb, bs, D).transpose(0, 2, 1, 3, 4).reshape(B * mb, H_kv, bs, D)
    table = np.arange(B * mb).reshape(B, mb)
    lens = [5, 16, 8]
    got = orc.gqa_paged(q, kp, vp, table, lens)
    for b, n in enumerate(lens):
        ref = orc.gqa(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n])
        np.testing.assert_allclose(got[b:b + 1], ref, rtol=1e-13, atol=1e-14)


def pin_paged_block_permutation(orc):
    """Moving blocks around the pool and renaming them in the table changes
    nothing, bit for bit; a shared block serves two sequences."""
    q, kp, vp, table, lens = rand_paged(63, 2, 4, 2, 4, 4, [10, 6], max_blocks=3)
    table[1, 0] = table[0, 0]                 # sequence 1 shares sequence 0's first block
    base = orc.gqa_paged(q, kp, vp, table, lens)
    perm = rng(64).permutation(kp.shape[0])   # new position of each block
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1)
    assert np.array_equal(orc.gqa_paged(q, kp2, vp2, table2, lens), base)
    shared = brute_force_paged(q, kp, vp, table, lens)
    np.testing.assert_allclose(base, shared, rtol=1e-12, atol=1e-13)


def pin_band_causal_is_causal(orc):
    """The band with no left limit and right edge 0 at offset 0 is the causal
    rule, bit for bit; with both sides open it is no mask at all."""
    q, k, v = rand_qkv(70, 2, 4, 2, 7, 9, 4)
    assert np.array_equal(orc.gqa_band(q, k, v, None, 0, -1, 0), orc.gqa(q, k, v, causal=True))
    assert np.array_equal(orc.gqa_band(q, k, v, None, 3, -1, -1), orc.gqa(q, k, v))


def pin_band_bottom_right_is_a_chunk(orc):
    """N queries placed at the end of M keys (offset M - N, causal) are the
    last N rows of causal self-attention over all M positions."""
    B, H, H_kv, M, N, D = 2, 6, 3, 11, 4, 8
    r = rng(71)
    q_full = r.standard_normal((B, H, M, D))
    k = r.standard_normal((B, H_kv, M, D))
    v = r.standard_normal((B, H_kv, M, D))
    full = orc.gqa(q_full, k, v, causal=True)
    chunk = orc.gqa_band(q_full[:, :, M - N:], k, v, None, M - N, -1, 0)
    np.testing.assert_allclose(chunk, full[:, :, M - N:], rtol=1e-13, atol=1e-14)
    # a single query at the end is plain decode over every key
    dec = orc.gqa_band(q_full[:, :, M - 1:], k, v, None, M - 1, -1, 0)
    np.testing.assert_allclose(dec, orc.gqa(q_full[:, :, M - 1:], k, v), rtol=1e-13, atol=1e-14)


def pin_band_brute_force(orc):
    """Sliding windows and two-sided bands against pure-Python loops, with a
    mask on top and offsets that leave some rows empty (NaN)."""
    B, H, H_kv, N, M, D = 2, 4, 2, 6, 9, 4
    q, k, v = rand_qkv(72, B, H, H_kv, N, M, D)
    extra = rng(73).random((B, N, M)) < 0.8
    for q_off, wl, wr in [(0, 2, 0), (3, 1, 1), (-2, 0, 3), (5, -1, 2), (0, 3, -1), (-8, -1, 0)]:
        mask = [[[bool(extra[b][i][j]) and (wl < 0 or j >= i + q_off - wl)
                  and (wr < 0 or j <= i + q_off + wr)
                  for j in range(M)] for i in range(N)] for b in range(B)]
        got = orc.gqa_band(q, k, v, extra, q_off, wl, wr)
        ref = brute_force(q, k, v, mask)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def pin_band_wide_window_is_causal(orc):
    """A window at least as long as the keys changes nothing."""
    q, k, v = rand_qkv(74, 1, 4, 1, 8, 8, 4)
    np.testing.assert_allclose(orc.gqa_band(q, k, v, None, 0, 8, 0),
                               orc.gqa(q, k, v, causal=True), rtol=0, atol=0)


def pin_band_window_width(orc):
    """The width of the band, counted without restating its inequalities.
    With K = 0 every visible key gets the same weight (pin_zero_keys_give_mean),
    so a V that holds the key index j in channel 0 and j^2 in channel 1 makes
    the output the mean and the mean square of the visible key indices.  The
    W consecutive integers a .. a+W-1 have mean a + (W-1)/2 and variance
    (W^2 - 1)/12, so an interior row with window_left = W - 1 and right edge
    0 (W keys ending at its position p = i + q_offset) must give mean
    p - (W-1)/2 and variance (W^2-1)/12, and a two-sided band (wl, wr) must
    give W = wl + wr + 1 keys centred at p + (wr - wl)/2."""
    N, M, D = 12, 40, 2
    j = np.arange(M, dtype=np.float64)
    v = np.stack([j, j * j], axis=-1)[None, None]              # [1, 1, M, 2]
    k = np.zeros((1, 1, M, D))
    q = rng(75).standard_normal((1, 2, N, D))
    for q_off, wl, wr in [(20, 0, 0), (20, 1, 0), (20, 4, 0), (20, 7, 0), (15, 2, 3),
                          (10, 0, 5), (25, 6, 6)]:
        out = orc.gqa_band(q, k, v, None, q_off, wl, wr)
        W = wl + wr + 1
        for i in range(N):
            p = i + q_off
            if p - wl < 0 or p + wr >= M:
                continue                       # not an interior row
            mean = out[0, 0, i, 0]
            var = out[0, 0, i, 1] - mean * mean
            assert abs(mean - (p + (wr - wl) / 2)) < 1e-9, (q_off, wl, wr, i, mean)
            assert abs(var - (W * W - 1) / 12) < 1e-7, (q_off, wl, wr, i, var)


PINS = [pin_worked_example_shape, pin_library_crosscheck, pin_brute_force,
        pin_mha_equals_per_head, pin_mqa_brute_force, pin_single_key,
        pin_two_keys_closed_form, pin_scale_exact, pin_zero_keys_give_mean,
        pin_head_mapping_exact, pin_weights_sum_to_one,
        pin_masked_keys_contribute_nothing, pin_causal_properties,
        pin_key_permutation, pin_empty_row_is_nan, pin_rejects_bad_group,
        pin_paged_brute_force, pin_paged_identity_table, pin_paged_length_is_truncation,
        pin_paged_block_permutation, pin_band_causal_is_causal,
        pin_band_bottom_right_is_a_chunk, pin_band_brute_force, pin_band_wide_window_is_causal,
        pin_band_window_width]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(gqa_oracle)


def test_tiling_differs():
    """The tiled head mapping used by one page (K.repeat over heads) gives a
    different answer whenever 1 < H_kv < H, so the two readings are
    distinguishable on random inputs."""
    for H, H_kv in [(4, 2), (8, 2), (6, 3), (8, 4)]:
        q, k, v = rand_qkv(40 + H, 1, H, H_kv, 4, 6, 8)
        g = H // H_kv
        tiled = oracle.gqa(q, np.tile(k, (1, g, 1, 1)), np.tile(v, (1, g, 1, 1)))
        inter = oracle.gqa(q, k, v)
        assert np.max(np.abs(tiled - inter)) > 1e-3
    # g == 1 or H_kv == 1: the two mappings coincide
    q, k, v = rand_qkv(50, 1, 4, 1, 3, 5, 4)
    np.testing.assert_allclose(oracle.gqa(q, np.tile(k, (1, 4, 1, 1)),
                                          np.tile(v, (1, 4, 1, 1))),
                               oracle.gqa(q, k, v), rtol=1e-14)


# ------------------------------------------------------- planted mistakes
MUTANTS = {
    "tile_instead_of_interleave": (r"np\.repeat\(x, group, axis=1\)",
                                   "np.tile(x, (1, group, 1, 1))"),
    "no_scale": (r" / math\.sqrt\(D\)", ""),
    "scale_by_D": (r"math\.sqrt\(D\)", "D"),
    "causal_strict": (r"\(j <= i\)", "(j < i)"),
    "causal_transposed": (r"\(j <= i\)", "(j >= i)"),
    "mask_polarity": (r"vis &= np\.asarray\(mask, dtype=bool\)",
                      "vis &= ~np.asarray(mask, dtype=bool)"),
    "softmax_wrong_axis": (r"e / e\.sum\(axis=-1, keepdims=True\)",
                           "e / e.sum(axis=-2, keepdims=True)"),
    "v_from_k": (r"vb = expand_kv\(np\.asarray\(v\[", "vb = expand_kv(np.asarray(k["),
    "group_from_kv": (r"return H // H_kv", "return max(1, H_kv // H)"),
    "max_not_subtracted_wrong_sign": (r"np\.exp\(scores - row_max\)",
                                      "np.exp(row_max - scores)"),
    "mask_ignored": (r"vis &= np\.asarray\(mask, dtype=bool\)", "pass"),
    "transposed_v": (r"out\[b\] = np\.matmul\(w, vb\)",
                     "out[b] = np.matmul(w, vb.transpose(0, 2, 1)[:, :w.shape[-1], :]) if vb.shape[1] == vb.shape[2] else np.matmul(w, vb)[..., ::-1]"),
    "paged_row_offset": (r"k_pool\[blk, :, t % bs, :\]", "k_pool[blk, :, (t + 1) % bs, :]"),
    "paged_block_index": (r"table\[b, t // bs\]", "table[b, t % max_blocks]"),
    "paged_length_inclusive": (r"for t in range\(n\):", "for t in range(min(n + 1, M)):"),
    "paged_v_from_k": (r"v\[b, :, t, :\] = v_pool", "v[b, :, t, :] = k_pool"),
    "band_left_strict": (r"vis &= j >= pos - window_left", "vis &= j > pos - window_left"),
    "band_right_strict": (r"vis &= j <= pos \+ window_right", "vis &= j < pos + window_right"),
    "band_offset_sign": (r"pos = i \+ q_offset", "pos = i - q_offset"),
    "band_mask_dropped": (r"vis = vis & np\.asarray\(mask, dtype=bool\)", "vis = vis"),
    "paged_head_ignored": (r"k\[b, :, t, :\] = k_pool\[blk, :,", "k[b, :, t, :] = k_pool[blk, :1,"),
}


def _mutant(name):
    pat, rep = MUTANTS[name]
    src = open(gqa_oracle.__file__).read()
    new, n = re.subn(pat, rep, src)
    assert n >= 1, f"mutation {name} did not apply"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(new, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception:          # noqa: BLE001 - any failure counts
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
