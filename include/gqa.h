/*
 * gqa.h - C ABI of the grouped-query attention forward library (libgqa.so),
 * built for AMD Instinct MI355X (gfx950).
 *
 * Operation (all entry points): for every batch row b, query head h and
 * query position i,
 *
 *     O[b,h,i,:] = sum_j softmax_j( Q[b,h,i,:] . K[b,h/g,j,:] / sqrt(D) ) V[b,h/g,j,:]
 *
 * with g = H / H_kv query heads per KV head, i.e. query head h reads KV head
 * h / g (integer division).  That is the repeat-interleave grouping of
 * "28. Grouped-Query Attention (GQA)" (sections *Problem*, *Step-by-Step
 * Approach*, *Reference solution*) and the [B,H,N,D] / [B,H_kv,M,D] interface
 * of "Multi-Query Attention" (section *Implementation*), where a real kernel
 * expresses the grouping as a zero stride over the head dimension instead of
 * materialising the expansion.  The group size comes from the shapes; there is
 * no separate group argument.
 *
 * The softmax runs over the keys that are visible to query i:
 *   - mask (optional, may be NULL): uint8 [B, N, M], nonzero = key visible,
 *     the same for every head (the reference solution's boolean mask, which
 *     is broadcast over heads and sets invisible scores to -inf);
 *   - causal (prefill only): key j visible to query i iff j <= i, for any N
 *     and M (top-left aligned; the self-attention causal mask of "Grouped-Query
 *     Attention Explained Simply", *Minimal implementation*).
 *   Mask and causal combine by AND.  A query row that sees no key yields NaN
 *   in every output element of that row (the reference recipe's softmax over
 *   all -inf scores).
 *
 * Layouts: contiguous row-major.  q [B,H,N,D], k and v [B,H_kv,M,D],
 * out [B,H,N,D].  Scale is fixed at 1/sqrt(D).  Accumulation is fp32.
 *
 * Supported: all dims >= 1, H % H_kv == 0, 1 <= D <= 256,
 * D * sizeof(in_dtype) a multiple of 16 bytes (bf16 and fp16: D % 8 == 0;
 * fp32: D % 4 == 0).  q, k, v, out and workspace must be 16-byte aligned.
 * in_dtype is the type of q, k and v; out_dtype is in_dtype or GQA_F32.
 * 16-bit inputs (bf16, fp16) run on the 16-bit matrix cores; the softmax
 * weights are rounded to the input type for the P.V product, everything
 * else accumulates in fp32.  fp16 is the cache precision named by the
 * KV-cache figure of "Multi-Query Attention" (after *Implementation*).
 * Element counts must fit in a signed 64-bit integer and B*H*N, B*H_kv*M
 * must each stay below 2^31 rows.
 *
 * Ownership: every pointer is device memory owned by the caller.  The
 * library never allocates, frees or keeps a pointer past the call.  out must
 * not overlap q, k, v, mask or workspace.
 *
 * Synchronisation and errors: calls are asynchronous.  They return after
 * enqueueing work on `stream` (a hipStream_t passed as void*; NULL is the
 * default stream).  Every argument check runs on the host before any HIP call,
 * so a rejected call has no side effect.  The library never aborts and never
 * prints.  Calls on different streams are independent as long as each decode
 * call uses its own workspace.
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In C++ the enums below get int as their fixed underlying type, so that any
 * int a C caller passes is a valid value (the library reports an unknown
 * code as an error instead of reading an out-of-range enum).  The layout is
 * the same as C's int-sized enums. */
#ifdef __cplusplus
#define GQA_ENUM_BASE : int
#else
#define GQA_ENUM_BASE
#endif

/* Size of the counter area at the start of a decode workspace. */
#define GQA_DECODE_COUNTER_BYTES 16384

/* Size of the fixed per-GPU scratch area of gqa_decode_noalloc (16 MiB). */
#define GQA_DECODE_NOALLOC_SCRATCH_BYTES (16u << 20)

typedef enum GQA_ENUM_BASE {
  GQA_OK = 0,
  GQA_ERR_NULL = 1,        /* a required pointer is NULL                      */
  GQA_ERR_SHAPE = 2,       /* a dimension < 1, or sizes overflow the limits   */
  GQA_ERR_GROUP = 3,       /* H is not a multiple of H_kv                     */
  GQA_ERR_DTYPE = 4,       /* unknown dtype, or out_dtype not in {in, F32}    */
  GQA_ERR_ALIGN = 5,       /* q/k/v/out/workspace not 16-byte aligned         */
  GQA_ERR_UNSUPPORTED = 6, /* D > 256, D*sizeof(in_dtype) % 16 != 0, or a
                              paged block_size that is not a multiple of 16  */
  GQA_ERR_WORKSPACE = 7,   /* decode workspace missing or too small           */
  GQA_ERR_HIP = 8,         /* the HIP runtime reported a launch error         */
  GQA_ERR_ALIAS = 9,       /* out overlaps an input or the workspace          */
  GQA_ERR_SCRATCH = 10     /* gqa_decode_noalloc: the problem needs more than
                              GQA_DECODE_NOALLOC_SCRATCH_BYTES of scratch    */
} gqa_status_t;

typedef enum GQA_ENUM_BASE {
  GQA_F32 = 0,  /* IEEE binary32                                              */
  GQA_BF16 = 1, /* bfloat16; outputs are rounded to nearest, ties to even     */
  GQA_F16 = 2   /* IEEE binary16 (half); outputs rounded to nearest even      */
} gqa_dtype_t;

/*
 * Decode: one query position per (batch row, head), N = 1.  This is the
 * autoregressive step that re-reads the whole KV cache (the bandwidth-bound
 * case of "Multi-Query Attention", *Theory*; "Grouped-Query Attention
 * Explained Simply", Q/A on why decode is memory-bandwidth bound).
 *
 *   q    [B, H, 1, D]     in_dtype
 *   k, v [B, H_kv, M, D]  in_dtype (the KV cache, M cached positions)
 *   mask [B, 1, M] uint8 or NULL (nonzero = key visible)
 *   out  [B, H, 1, D]     out_dtype
 *   workspace: device buffer of at least gqa_decode_workspace_size(...)
 *     bytes (may be NULL when that size is 0).  Its first
 *     GQA_DECODE_COUNTER_BYTES bytes are arrival counters, one per unit of
 *     work whose keys are split over several workgroups: once the last
 *     split of a unit has arrived, the unit's fp32 partial results, which
 *     follow the counters, are merged (by that split, or with more than 32
 *     query heads per KV head by all of the unit's splits, each a slice of
 *     its heads).  The counter area MUST be zero before the first call
 *     (zero the buffer once after allocating it); every call, of any shape
 *     and through either decode entry point, leaves it zero again, so one
 *     buffer serves every later call on the same stream that fits in it.
 *     The rest needs no initialisation.  Nonzero counters give wrong
 *     outputs (no error is reported).  Two calls that may run at the same
 *     time (different streams) need two workspaces.
 * The result is deterministic: the same inputs give bit-identical outputs
 * (the splits are always merged in split order, whichever finishes last).
 */
gqa_status_t gqa_decode(const void* q, const void* k, const void* v,
                        const uint8_t* mask, void* out,
                        int B, int H, int H_kv, int M, int D,
                        gqa_dtype_t in_dtype, gqa_dtype_t out_dtype,
                        void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Decode without allocation or workspace: for callers that cannot allocate
 * device memory at call time (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same operation, arguments,
 * layouts, results (bit for bit) and errors as gqa_decode, except that the
 * key-split partials and arrival counters live in a fixed scratch area that
 * the library holds on each GPU it runs on, from the first call on that GPU
 * until the process ends: GQA_DECODE_NOALLOC_SCRATCH_BYTES (16 MiB) of
 * device memory.  No call allocates or frees anything.
 *   - Problems whose gqa_decode_workspace_size(...) exceeds that size are
 *     rejected with GQA_ERR_SCRATCH before any HIP call.
 *   - The first call on a GPU looks up the scratch area and clears its
 *     counters with a small kernel on `stream`, ahead of the decode.
 *   - Every call on one GPU uses the same scratch area, and each call leaves
 *     the counters zero for the next one.  Calls that may overlap on one GPU
 *     (different streams, or graphs replayed concurrently) race on it and
 *     give wrong results: serialise them, or use gqa_decode with one
 *     workspace per stream.
 */
gqa_status_t gqa_decode_noalloc(const void* q, const void* k, const void* v,
                                const uint8_t* mask, void* out,
                                int B, int H, int H_kv, int M, int D,
                                gqa_dtype_t in_dtype, gqa_dtype_t out_dtype,
                                void* stream);

/*
 * Bytes of decode workspace for these sizes (independent of dtype and of
 * the device).  Returns 0 when no workspace is needed or when the sizes are
 * invalid (gqa_decode then reports the size error).
 */
size_t gqa_decode_workspace_size(int B, int H, int H_kv, int M, int D);

/*
 * Paged decode: the decode above over a KV cache kept in fixed-size blocks,
 * with one cache length per sequence.  This is the serving form of the
 * KV cache whose per-sequence size the grouping shrinks ("Grouped-Query
 * Attention vs Multi-Head Attention: Understanding GQA Implementation",
 * sections on the KV-cache buffers and *Summary*; "Multi-Query Attention",
 * *Theory* on the decode step re-reading the cache).
 *
 *   q           [B, H, 1, D]                          in_dtype
 *   k_pool,
 *   v_pool      [num_blocks, H_kv, block_size, D]     in_dtype
 *   block_table [B, max_blocks] int32: block_table[b][t] is the pool block
 *               that holds keys t*block_size ... (t+1)*block_size - 1 of
 *               sequence b
 *   kv_len      [B] int32: sequence b has keys 0 .. kv_len[b]-1 (values are
 *               clamped to [0, max_blocks*block_size]; entries of the table
 *               past the last used block are never read)
 *   out         [B, H, 1, D]                          out_dtype
 *   workspace   at least gqa_decode_paged_workspace_size(...) bytes, with
 *               the same rules as for gqa_decode (counter area zero before
 *               the first call, left zero by every call)
 * Key t of sequence b and KV head j is row
 *   k_pool[block_table[b][t / block_size], j, t % block_size, :].
 * A sequence with kv_len[b] == 0 sees no key and yields NaN.  The result
 * equals gqa_decode over the gathered cache [B, H_kv, max_blocks*block_size,
 * D] with mask[b][0][t] = (t < kv_len[b]).
 * Work split: when the batch has fewer than 4096 (batch row, KV head, head
 * chunk) units and more than 256 cached key slots, each unit's keys are cut
 * into pieces balanced over the actual lengths (planned on the device from
 * kv_len), merged in piece order.  Results are deterministic for given
 * lengths.
 * Supported: block_size a positive multiple of 16 (else
 * GQA_ERR_UNSUPPORTED); the limits of gqa_decode with M = max_blocks *
 * block_size; block_table and kv_len are device memory, 4-byte aligned.
 * Block ids are trusted: an id outside [0, num_blocks) is clamped into that
 * range (memory stays in bounds, the result is then meaningless).  Several
 * sequences may share a block.  No mask argument: kv_len is the visibility.
 */
gqa_status_t gqa_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_table, const int32_t* kv_len,
                              void* out, int B, int H, int H_kv, int max_blocks,
                              int block_size, int num_blocks, int D,
                              gqa_dtype_t in_dtype, gqa_dtype_t out_dtype,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/* Bytes of paged-decode workspace for these sizes (independent of dtype,
 * of the lengths and of the device); 0 when none is needed or the sizes are
 * invalid. */
size_t gqa_decode_paged_workspace_size(int B, int H, int H_kv, int max_blocks,
                                       int block_size, int D);

/*
 * Prefill: N query positions per (batch row, head) against M keys, with an
 * optional mask and causal flag (the self-attention forward of "Grouped-Query
 * Attention Explained Simply", *Minimal implementation*, and the masked
 * forward of the reference solution of "28. Grouped-Query Attention (GQA)").
 *
 *   q    [B, H, N, D]     in_dtype
 *   k, v [B, H_kv, M, D]  in_dtype
 *   mask [B, N, M] uint8 or NULL (nonzero = key visible)
 *   causal: 0 or 1 (nonzero): key j visible to query i iff j <= i
 *   out  [B, H, N, D]     out_dtype
 * No workspace.  Deterministic.
 */
gqa_status_t gqa_prefill(const void* q, const void* k, const void* v,
                         const uint8_t* mask, int causal, void* out,
                         int B, int H, int H_kv, int N, int M, int D,
                         gqa_dtype_t in_dtype, gqa_dtype_t out_dtype,
                         void* stream);

/*
 * Banded prefill: gqa_prefill with the visible keys of query i limited to a
 * band around its position i + q_offset in the key sequence:
 *
 *   key j visible  iff  (window_left  < 0 || j >= i + q_offset - window_left)
 *                   and (window_right < 0 || j <= i + q_offset + window_right)
 *                   and (mask == NULL || mask[b][i][j] != 0).
 *
 * A negative window leaves that side unbounded.  Special cases:
 *   window_left < 0, window_right = 0, q_offset = 0      causal (= gqa_prefill
 *                                                          with causal = 1)
 *   window_left < 0, window_right = 0, q_offset = M - N  bottom-right causal:
 *       the N queries are the last N positions of the M keys (a prefill
 *       chunk appended to a cache of M - N earlier keys)
 *   window_left = W - 1, window_right = 0                 sliding window of W
 *       keys ending at the query's own position, the local attention that
 *       "28. Grouped-Query Attention (GQA)" (*Problem*) mentions Mistral
 *       using alongside GQA.
 * Key tiles outside every row's band are skipped, so the work is that of the
 * visible pairs.  Rows that see no key yield NaN.  Same layouts, dtypes,
 * limits and errors as gqa_prefill; any int q_offset and windows are valid.
 */
gqa_status_t gqa_prefill_band(const void* q, const void* k, const void* v,
                              const uint8_t* mask, void* out,
                              int B, int H, int H_kv, int N, int M, int D,
                              int q_offset, int window_left, int window_right,
                              gqa_dtype_t in_dtype, gqa_dtype_t out_dtype,
                              void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* gqa_status_string(gqa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */
