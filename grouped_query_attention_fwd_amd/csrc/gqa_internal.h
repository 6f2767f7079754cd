// Host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

// Arguments after validation.  Sizes are the caller's; derived values
// (group size, padded head dim, split count) are filled by the ABI layer.
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* mask;  // [B, 1, M] or null
  void* out;
  // [units][splits][16][D + 4] fp32 (with paged pieces: [pieces][16][D + 4],
  // a unit's pieces consecutive), or null when splits == 1
  float* partials;
  // [units] arrival counters (splits > 1), zero between calls: the last
  // split of a unit to finish resets its counter and merges the unit
  unsigned* counters;
  // paged KV (block_table != null): k/v are pools [num_blocks][H_kv][block_size][D];
  // key j of sequence b lives in block block_table[b * max_blocks + j / block_size]
  // at row j % block_size, and only keys j < kv_len[b] exist.  M = max_blocks * block_size.
  const int32_t* block_table;
  const int32_t* kv_len;
  int num_blocks, block_size, max_blocks;
  int B, H, H_kv, M, D;
  int g;                // H / H_kv
  int head_chunk;       // query heads per unit (<= 16)
  int head_chunks;      // ceil(g / head_chunk): units per (b, KV head)
  int xcd_group;        // 1: the head chunks of one (b, KV head) share an XCD
  int splits;           // key-range splits per unit
  int keys_per_split;   // multiple of 256
  // paged only: > 0 launches this many workgroups, which split the keys in
  // pieces balanced over the actual lengths (planned in the kernel)
  int pieces;
  int rotate;           // 1: each workgroup starts its key walk at its own round
  int in_type;          // element type of q, k, v: kF32, kBF16 or kF16
  bool out_f32;
  // timing build only (GQA_DECODE_TRACE): per-workgroup records, else null
  unsigned long long* trace;
};

// Timing build: workgroup records of the decode trace (8 words each).
constexpr int kTraceRecords = 8192;

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* mask;  // [B, N, M] or null
  void* out;
  int B, H, H_kv, N, M, D;
  int g;
  // Band: key j is visible to query i iff
  //   (wl < 0 || j >= i + q_offset - wl) && (wr < 0 || j <= i + q_offset + wr).
  // Causal (top-left) is q_offset = 0, wl = -1, wr = 0.
  int q_offset, wl, wr;
  // mask strides in bytes: rows M and batch rows N * M for a [B, N, M]
  // mask; rows 0 and batch rows M when one [B, 1, M] row serves every query
  int mask_rs;
  long long mask_bs;
  // key splits: with splits > 1 workgroup column s covers keys
  // [s * kps, (s + 1) * kps) (kps a multiple of 64) and writes a partial
  // (m, l, acc) per query row to partials [B * H * N][splits][D + 4] fp32;
  // the splits of a position block then merge them among themselves
  // (counters: arrival counters and slice claims, zero between calls) or a
  // second kernel merges them (counters null, or the launch does not allow
  // the in-kernel merge)
  int splits, kps;
  float* partials;
  unsigned* counters;
  int rows16;           // 1: 16 query rows per wave (the decode of large groups)
  int in_type;          // element type of q, k, v: kF32, kBF16 or kF16
  bool out_f32;
};

// Largest grid x dimension a launch uses (a multiple of the 8 XCDs, so the
// XCD of workgroup L = x + kMaxGridX * z stays L % 8).  Launches with more
// workgroups fold the rest into grid z; the kernels rebuild L from both and
// drop the workgroups past the end.  This keeps every grid dimension far
// below the runtime's limit of 2^32 work-items.
constexpr unsigned kMaxGridX = 1u << 16;
inline dim3 fold_grid(long n, unsigned y) {
  const unsigned x = n > (long)kMaxGridX ? kMaxGridX : (unsigned)n;
  const unsigned z = (unsigned)((n + x - 1) / x);
  return dim3(x, y, z);
}

// Decode workspace layout: kCounterBytes of arrival counters (one per unit,
// zero between calls), then the split partials.  The counter area has the
// same place and size for every plan, so partials never land on it.
constexpr size_t kCounterBytes = 16384;
constexpr int kMaxCounters = (int)(kCounterBytes / 4);

// Split plan shared by the workspace query and the decode launch, so both
// agree for the same shapes.
struct DecodePlan {
  // wide: large groups (more than 32 heads) run as a prefill with the group's
  // heads as query rows (one shared K/V tile stream per (b, KV head)), split
  // over keys into wide_splits ranges of wide_kps keys
  int wide, wide_splits, wide_kps;
  int head_chunk;
  int head_chunks;
  int xcd_group;
  int splits;
  int keys_per_split;
  int pieces;              // paged: length-balanced pieces (0: static splits)
  size_t partials_bytes;
  size_t workspace_bytes;  // kCounterBytes + partials_bytes; 0 when splits == 1
};
DecodePlan plan_decode(int B, int H, int H_kv, int M, int D, bool paged);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

}  // namespace gqa
