// Decode (one query position) grouped-query attention forward for gfx950.
//
// Operation: for each batch row b and query head h,
//   o[b,h,:] = softmax_j(q[b,h,:] . k[b,h/g,j,:] / sqrt(D)) v[b,h/g,j,:]
// ("28. Grouped-Query Attention (GQA)", *Reference solution*, with the
// grouping done as a zero head stride as "Multi-Query Attention",
// *Implementation*, describes for real kernels).
//
// Why it is shaped this way: decode re-reads the whole KV cache once per
// step and does ~g flop per byte ("Multi-Query Attention", *Theory*), so the
// kernel is HBM-bound.  Each K and V row is read from HBM exactly once and
// used for all the query heads of its group (up to 16 per workgroup).
//
// Work split: one workgroup of four waves per (batch row, KV head, chunk of
// up to 16 query heads, key range).  The key ranges are equal splits, or,
// for a paged batch, pieces balanced over the sequences' actual lengths,
// planned by every workgroup from kv_len.  Inside a workgroup the waves
// take interleaved chunks of KC keys, addressed per aligned group of 16 keys
// (contiguous rows, or one block-table entry of a paged cache, in which case
// each sequence's own length ends its key range).  Per chunk a wave
//   1. loads K rows straight into MFMA operand registers (16 bytes per lane)
//      and V rows with coalesced 16-byte loads, non-temporal (each byte is
//      read once per call; the hint measured 10-12 % faster), all issued up front with
//      clamped (always valid) addresses so nothing waits on a branch, one
//      chunk ahead of the math (two register buffers used in turn; a paged
//      cache's block-table entries are read one chunk further ahead);
//   2. forms S^T = K Q^T on the matrix cores (keys x heads);
//   3. copies the V chunk into its private, XOR-swizzled LDS area;
//   4. runs the online softmax with scores scaled by log2(e)/sqrt(D) and the
//      hardware exp2; lane l%16 owns head l%16, so the running max and the
//      rescale factor stay in the lane and the row max needs two cross-lane
//      steps;
//   5. forms O^T += V^T P^T on the matrix cores, reading V^T from LDS with
//      the transposing ds_read_b64_tr_b16 (16-bit) or plain reads (fp32).
// The four waves merge (m, l, acc) through LDS.  With one split the result is
// written directly.  Otherwise every workgroup stores its (m, l, acc) partial
// to the fp32 workspace and takes a ticket from the unit's arrival counter;
// the workgroup that arrives last merges the unit's splits in split order
// (so the result is bit-reproducible whichever finishes last) and sets the
// counter back to zero for the next call.
// Groups of more than 32 heads (contiguous cache) go through the prefill
// kernel instead, with the heads as query rows (see plan_decode).
#include "gqa_device.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

// 1: the timing build.  Every workgroup writes one record to a.trace:
// wall-clock ticks at its start, when all its waves have finished their
// keys, after its arrival ticket and at its end, where it ran (XCD, shader
// engine, CU), ticks once it knows its keys (after a paged piece plan), its
// grid position, and whether it merged.  Off in the
// library proper (no code at all).
#ifndef GQA_DECODE_TRACE
#define GQA_DECODE_TRACE 0
#endif

#ifndef GQA_DECODE_WAVES
#define GQA_DECODE_WAVES 4
#endif
constexpr int kWaves = GQA_DECODE_WAVES;  // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kRoundKeys = 256;  // keys_per_split is a multiple of this
// Workgroups to aim for when choosing the split count.
#ifndef GQA_DECODE_TARGET_WGS
#define GQA_DECODE_TARGET_WGS 256
#endif
// Groups of more than GQA_DECODE_WIDE_MIN_G heads through the prefill kernel
// (see plan_decode); measured: 11 % faster at g = 64, 4 % slower at g = 32
// than head chunks that re-read K/V.
#ifndef GQA_DECODE_WIDE
#define GQA_DECODE_WIDE 1
#endif
#ifndef GQA_DECODE_WIDE_MIN_G
#define GQA_DECODE_WIDE_MIN_G 32
#endif
#ifndef GQA_DECODE_WIDE_TARGET_WGS
#define GQA_DECODE_WIDE_TARGET_WGS 256
#endif
// The paged form launches this many workgroups for fewer units (two rounds
// of 256 CUs: with mixed lengths, shorter pieces even out the CUs' work;
// measured 33.4 against 35.7 us on the mixed-length Mistral-shaped batch).
// Near-equal lengths use only kPagedEvenWGs of them (below).
#ifndef GQA_DECODE_PAGED_TARGET_WGS
#define GQA_DECODE_PAGED_TARGET_WGS 512
#endif
static_assert(GQA_DECODE_TARGET_WGS <= kMaxCounters && GQA_DECODE_PAGED_TARGET_WGS <= kMaxCounters,
              "a split plan needs fewer units than the counter area holds");
static_assert(GQA_DECODE_PAGED_TARGET_WGS % 8 == 0, "the piece grid is a multiple of the XCD count");
// Pieces planned for near-equal lengths: one per CU.  Cutting them for two
// rounds of workgroups only adds restarts and merges (the full-length
// batch: 49.5 against 48.2 us).
constexpr int kPagedEvenWGs = 256;
// 1: a paged decode that splits keys cuts them into pieces balanced over
// the actual sequence lengths, planned in the kernel (GQA_DECODE_PAGED_
// TARGET_WGS workgroups); 0: the static split plan, sized for the longest
// possible sequence.
#ifndef GQA_DECODE_PAGED_PIECES
#define GQA_DECODE_PAGED_PIECES 1
#endif

template <bool H16, int DP>
struct DecCfg {
  static constexpr int ELT = H16 ? 2 : 4;
  // keys per wave chunk (bounded by LDS and by the registers of the loads)
  static constexpr int KC = H16 ? (DP <= 64 ? 64 : 32) : (DP <= 64 ? 64 : (DP == 128 ? 32 : 16));
  static constexpr int NKB = KC / 16;                 // 16-key MFMA blocks per chunk
  static constexpr int NDB = DP / 16;                 // 16-wide d blocks of O
  static constexpr int QCH = H16 ? DP / 32 : DP / 16;  // 16-byte Q/K chunks per lane per key
  static constexpr int CPR = DP * ELT / 16;           // 16-byte chunks per row
  static constexpr int ROWB = H16 ? DP * 2 : DP * 4 + 16;  // LDS row stride (fp32 rows padded)
  static constexpr int VBYTES = KC * ROWB;            // LDS bytes of one wave's V chunk
  static constexpr int VLOADS = KC * CPR / 64;        // 16-byte V loads per lane per chunk
  // the rows of one V load instruction lie in one aligned group of 16 keys
  static_assert(KC % 16 == 0 && 64 % CPR == 0 && 64 / CPR <= 16, "V load rows span a group");
  static constexpr int SPR = DP / 16;                 // 32-byte segments per 16-bit row
  static constexpr int SWZ = (SPR < 8 ? SPR : 8) - 1;
  // Registers of one chunk's loads; when two chunks fit, the next chunk is
  // loaded while the current one is computed.
  static constexpr int LOAD_VGPRS = (NKB * QCH + VLOADS) * 4;
  static constexpr bool PREFETCH = LOAD_VGPRS <= 64;
  static constexpr int COMBINE_BYTES = kWaves * 16 * DP * 4 + 2 * kWaves * 16 * 4;
  static constexpr int LDS_BYTES =
      (kWaves * VBYTES > COMBINE_BYTES) ? kWaves * VBYTES : COMBINE_BYTES;
};

// Byte offset of 16-byte chunk `chunk` of LDS row `row` of a V chunk.
template <bool H16, int DP>
__device__ __forceinline__ uint32_t v_off(int row, int chunk) {
  using C = DecCfg<H16, DP>;
  if constexpr (H16) {
    return row * C::ROWB + ((chunk ^ (2 * (row & C::SWZ))) << 4);
  } else {
    return row * C::ROWB + (chunk << 4);
  }
}

// Output element idx: fp32, or the 16-bit input type ET.
template <int ET, bool OUTF32>
__device__ __forceinline__ void store_out(void* out, size_t idx, float x) {
  if constexpr (OUTF32) {
    reinterpret_cast<float*>(out)[idx] = x;
  } else {
    static_assert(ET != kF32, "fp32 inputs have fp32 outputs");
    reinterpret_cast<uint16_t*>(out)[idx] = cvt16<ET>(x);
  }
}

// Four consecutive output elements idx .. idx + 3 (idx a multiple of 4).
template <int ET, bool OUTF32>
__device__ __forceinline__ void store_out4(void* out, size_t idx, f32x4 x) {
  if constexpr (OUTF32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + idx) = x;
  } else {
    const u32x2 pk = {pack16<ET>(x[0], x[1]), pack16<ET>(x[2], x[3])};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + idx) = pk;
  }
}

// Key-split partials of one unit: [splits][16 heads][D + 4] fp32 rows of
// (m, l, -, -, acc[0..D)), m being the score maximum (unscaled) the weights
// were taken against.  Byte offset of row (split, head):
__device__ __forceinline__ uint32_t part_row(int split, int hh, int D) {
  return (uint32_t)((split * 16 + hh) * (D + 4)) * 4u;
}

// Merge the key-split partials of one (batch row, KV head, head chunk):
// m* = max_s m_s, o = sum_s acc_s 2^((m_s - m*) sl) / sum_s l_s 2^((m_s - m*) sl),
// taken over the splits in order, SB splits per memory round trip with a
// running m*, so the result does not depend on which split finished last.
// A thread owns quads (head, 4 consecutive d) tid, tid + kThreads, ...,
// QPT of them per round trip; every load of a round trip is issued before
// any of its arithmetic.
template <int ET, bool OUTF32, int QPT, int SB>
__device__ __forceinline__ void merge_quads(const DecodeArgs& a, __amdgpu_buffer_rsrc_t prs, int S,
                                            int b, int h0, int gh, int tid) {
  const int D = a.D, DQ = a.D >> 2;
  const int nq = gh * DQ;
  const float sl = kLog2e / sqrtf((float)D);
  for (int q0 = tid; q0 < nq; q0 += QPT * kThreads) {
    int hh[QPT], d[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int q = min(q0 + i * kThreads, nq - 1);  // clamped: loads stay valid
      hh[i] = q / DQ;
      d[i] = 4 * (q - hh[i] * DQ);
    }
    float mx[QPT], L[QPT];
    f32x4 A[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      mx[i] = kNegInf;
      L[i] = 0.f;
      A[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int s0 = 0; s0 < S; s0 += SB) {
      f32x2 ml[QPT][SB];
      f32x4 pa[QPT][SB];
#pragma unroll
      for (int i = 0; i < QPT; ++i) {
#pragma unroll
        for (int u = 0; u < SB; ++u) {
          const uint32_t ro = part_row(min(s0 + u, S - 1), hh[i], D);
          ml[i][u] = ld_dev2(prs, ro);
          pa[i][u] = ld_dev4(prs, ro + 16 + 4 * d[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < QPT; ++i) {
        float cm = kNegInf;
#pragma unroll
        for (int u = 0; u < SB; ++u) cm = fmaxf(cm, ml[i][u][0]);  // clamped copies change nothing
        const float nm = fmaxf(mx[i], cm);
        if (nm != kNegInf) {  // else nothing visible yet
          const float f0 = (mx[i] == kNegInf) ? 0.f : exp2_hw((mx[i] - nm) * sl);
          L[i] *= f0;
          A[i] *= f0;
#pragma unroll
          for (int u = 0; u < SB; ++u) {
            if (s0 + u < S) {
              const float f = exp2_hw((ml[i][u][0] - nm) * sl);
              L[i] = fmaf(ml[i][u][1], f, L[i]);
#pragma unroll
              for (int e = 0; e < 4; ++e) A[i][e] = fmaf(pa[i][u][e], f, A[i][e]);
            }
          }
          mx[i] = nm;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      if (q0 + i * kThreads < nq)
        store_out4<ET, OUTF32>(a.out, ((size_t)b * a.H + h0 + hh[i]) * D + d[i], A[i] / L[i]);
    }
  }
}

// Where a workgroup's keys lie: unit (b, KV head, head chunk), its split s
// of S, the index `first` of the unit's first partial, and keys
// [k_begin, k_end).
struct Piece {
  int unit, s, S, first, k_begin, k_end;
};

// Length-balanced pieces of a paged batch (a.pieces > 0): at most G =
// a.pieces workgroups, one per piece, with the longest piece as short as
// the lengths allow.  Unit u (b, KV head, head chunk) has n_u = ceil(len_b
// / 64) groups of 64 keys; with pieces of at most P groups it takes S_u =
// max(1, ceil(n_u / P)) pieces, and P is the smallest value with
// sum_u S_u <= G, found by bisection between ceil(N / G) and
// ceil(N / (G - U)) (N = sum_u n_u, U units; the upper end always fits,
// since sum_u S_u <= N / P + U).  Unit u's groups are then cut into S_u
// near-equal pieces.  Near-equal lengths skip the search: each unit is one
// piece (256 units or more) or floor(256 / U) pieces, one wave of
// workgroups.  Pieces are numbered unit by unit, units in
// order, and spread over the XCDs (below); workgroups left over have none.
// All units of batch row b share its length, so the sums run over batch
// rows, one wave reduction per 64 rows (kv_len is re-read from cache in
// each pass).  Every wave computes the plan itself; the result is
// wave-uniform.
__device__ __forceinline__ bool paged_piece(const DecodeArgs& a, int L, Piece& pc) {
  const int lane = threadIdx.x & 63;
  const int per_b = a.H_kv * a.head_chunks;
  const int U = a.B * per_b;
  const int G = a.pieces;
  const int rounds = (a.B + 63) >> 6;
  // clamped length of batch row lane + 64 r (0 past the last row); the
  // first 64 rows stay in a register, so the passes below do not wait on
  // a load each (a batch of more than 64 rows re-reads the rest from cache)
  auto len_of = [&](int b) { return b < a.B ? min(max(a.kv_len[b], 0), a.M) : 0; };
  const int len0 = len_of(lane);
  auto len_r = [&](int r) { return r == 0 ? len0 : len_of(lane + 64 * r); };
  int N = 0, nmax = 0;
  for (int r = 0; r < rounds; ++r) {
    const int n = (len_r(r) + 63) >> 6;
    N += n;
    nmax = max(nmax, n);
  }
  N = wave_sum(N) * per_b;  // the host keeps U * ceil(M / 64) below 2^30
  nmax = wave_max(nmax);
  // pieces of round r's batch row at piece size P (0 past the last row)
  auto pieces_of = [&](int r, int P) {
    const unsigned n = (unsigned)(len_r(r) + 63) >> 6;
    return lane + 64 * r < a.B ? (int)max(1u, (n + (unsigned)P - 1u) / (unsigned)P) : 0;
  };
  auto pieces_for = [&](int P) {
    int t = 0;
    for (int r = 0; r < rounds; ++r) t += pieces_of(r, P);
    return wave_sum(t) * per_b;
  };
  int lo = max(1, (N + G - 1) / G);
  int hi = max(lo, (N + (G - U) - 1) / (G - U));
  // Near-equal lengths (longest within 25 % of the mean) need no search.
  // With more units than one wave of workgroups, one piece per unit:
  // cutting them would only add a second round of workgroups and merges.
  // Otherwise floor(256 / U) pieces per unit (one wave of workgroups; the
  // rest of the G find no piece and return), P = ceil(nmax / that), which
  // fits G.
  if (4LL * nmax * U <= 5LL * N) {
    const int k = U >= kPagedEvenWGs ? 1 : min(G, kPagedEvenWGs) / U;
    lo = hi = max(1, (nmax + k - 1) / k);
  }
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (pieces_for(mid) <= G) hi = mid; else lo = mid + 1;
  }
  const int P = lo;
  // XCD-grouped order over the T pieces of the plan: workgroup L runs on XCD
  // L % 8 and takes piece (L % 8) * ceil(T / 8) + L / 8, so each XCD walks a
  // run of consecutive pieces (whole units, whose head chunks read the same
  // K/V rows, stay on one L2) and the XCDs get equal shares; workgroups past
  // an XCD's share have none.
  const int T = pieces_for(P);
  const int per = (T + 7) >> 3;
  if ((L >> 3) >= per) return false;
  const int i = (L & 7) * per + (L >> 3);
  if (i >= T) return false;
  int carry = 0;
  for (int r = 0; r < rounds; ++r) {
    const int b = lane + 64 * r;
    const int lb = len_r(r);
    const int sb = pieces_of(r, P);
    int incl = wave_incl_scan(sb * per_b) + carry;
    const int excl = incl - sb * per_b;
    const unsigned long long hit = __ballot(b < a.B && excl <= i && i < incl);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      const int S = __shfl(sb, src, 64);
      const int e0 = __shfl(excl, src, 64);
      const int blen = __shfl(lb, src, 64);
      const int nb = (blen + 63) >> 6;
      const int local = i - e0;
      const int ju = local / S;
      pc.unit = (64 * r + src) * per_b + ju;
      pc.s = local - ju * S;
      pc.S = S;
      pc.first = e0 + ju * S;
      if (pc.first + S > G) return false;  // never: the plan fits G (keeps partials in bounds)
      // near-equal cut of the unit's nb groups into S pieces
      pc.k_begin = min(64 * (int)(((long long)pc.s * nb) / S), blen);
      pc.k_end = min(64 * (int)(((long long)(pc.s + 1) * nb) / S), blen);
      return true;
    }
    carry = __shfl(incl, 63, 64);
  }
  return false;
}

// EXACT: D == DP, so no column of a row needs masking.  MASKED: a mask is
// given.  PAGED: K/V rows are found through a block table and each sequence
// has its own length.  NT: K/V loads carry the non-temporal hint; off when
// a unit's rows are read again by the unit of the group's next head chunk
// (the hint would evict them from L2 before that second read: g = 32 took
// 23.2 against 21.5 us with it).
template <int ET, int DP, bool EXACT, bool MASKED, bool PAGED, bool OUTF32, bool NT>
__global__ void __launch_bounds__(kThreads, 8 / kWaves) decode_kernel(DecodeArgs a) {
  constexpr bool H16 = ET != kF32;  // 16-bit elements: bf16 or fp16
  using C = DecCfg<H16, DP>;
  __shared__ __attribute__((aligned(16))) char smem_raw[C::LDS_BYTES];
#if GQA_DECODE_TRACE
  const unsigned long long tr_start = (unsigned long long)wall_clock64();
  unsigned long long tr_keys = 0, tr_ticket = 0, tr_plan = 0;
  const unsigned tr_wg = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  auto trace_out = [&](int merged) {
    if (threadIdx.x == 0 && a.trace != nullptr && tr_wg < (unsigned)kTraceRecords) {
      const unsigned xcc = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20);   // XCC_ID[3:0]
      const unsigned hw = __builtin_amdgcn_s_getreg((15 << 11) | (0 << 6) | 4);    // HW_ID[15:0]
      unsigned long long* r = a.trace + (size_t)tr_wg * 8;
      r[0] = tr_start;
      r[1] = tr_keys;
      r[2] = tr_ticket;
      r[3] = (unsigned long long)wall_clock64();
      r[4] = ((unsigned long long)xcc << 16) | hw;   // hw: CU in bits 11:8, SE in 14:13
      r[5] = tr_plan;
      r[6] = ((unsigned long long)blockIdx.x << 32) | blockIdx.y;
      r[7] = (unsigned long long)merged;
    }
  };
#endif
  lds_char* smem = (lds_char*)smem_raw;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int lane = tid & 63;
  const int c16 = lane & 15;
  const int qg = lane >> 4;

  // Units are numbered (b, KV head, head chunk).  With xcd_group the
  // workgroups are renumbered so that the head chunks of one (b, KV head),
  // which stream the same K/V rows, run side by side on one XCD (workgroup
  // L goes to XCD L % 8), where the later reader can find rows in L2.
  Piece pc;
  if (PAGED && a.pieces > 0) {
    if (!paged_piece(a, blockIdx.x, pc)) return;  // uniform: no piece for this workgroup
  } else {
    pc.unit = (int)(blockIdx.x + gridDim.x * blockIdx.z);
    if (pc.unit >= a.B * a.H_kv * a.head_chunks) return;  // past a folded grid's end (uniform)
    if (a.xcd_group) {
      const int x = pc.unit & 7, i = pc.unit >> 3;
      pc.unit = ((i / a.head_chunks) * 8 + x) * a.head_chunks + i % a.head_chunks;
    }
    pc.s = blockIdx.y;
    pc.S = a.splits;
    pc.first = pc.unit * a.splits;
    pc.k_begin = pc.s * a.keys_per_split;
    pc.k_end = min(a.M, pc.k_begin + a.keys_per_split);
  }
#if GQA_DECODE_TRACE
  tr_plan = (unsigned long long)wall_clock64();
#endif
  const int unit = __builtin_amdgcn_readfirstlane(pc.unit);
  const int s = __builtin_amdgcn_readfirstlane(pc.s);
  const int S = __builtin_amdgcn_readfirstlane(pc.S);
  const int per_b = a.H_kv * a.head_chunks;
  const int b = unit / per_b;
  const int rem = unit - b * per_b;
  const int j = rem / a.head_chunks;
  const int hc = rem - j * a.head_chunks;
  const int h0 = j * a.g + hc * a.head_chunk;
  const int gh = min(a.head_chunk, a.g - hc * a.head_chunk);
  const int D = EXACT ? DP : a.D;
  const int M = a.M;

  const int k_begin = __builtin_amdgcn_readfirstlane(pc.k_begin);
  int k_end = __builtin_amdgcn_readfirstlane(pc.k_end);
  if constexpr (PAGED) k_end = min(k_end, max(0, a.kv_len[b]));   // this sequence's keys

  // K/V rows are addressed per aligned group of 16 keys.  `group_off(g16, e)`
  // is the byte offset of the row of key g16 (a multiple of 16) inside the
  // K or V buffer; the other 15 keys of the group follow it contiguously.
  // The group start is wave-uniform, so a paged lookup is one scalar load.
  const size_t kv_base = PAGED ? 0 : ((size_t)b * a.H_kv + j) * (size_t)M * D;  // elements
  const char* kp = reinterpret_cast<const char*>(a.k) + kv_base * C::ELT;
  const char* vp = reinterpret_cast<const char*>(a.v) + kv_base * C::ELT;
  const int32_t* __restrict__ btab = PAGED ? a.block_table + (size_t)b * a.max_blocks : nullptr;
  // `entry` is the block-table entry of the group (paged only), read ahead
  // of time by tab_of below.
  auto group_off = [&](int g16, int entry) -> size_t {
    if constexpr (PAGED) {
      const int blk = g16 / a.block_size;
      // a block id outside the pool is clamped into it: memory stays safe,
      // the values are then the caller's responsibility
      const int phys = min(max(entry, 0), a.num_blocks - 1);
      return (((size_t)phys * a.H_kv + j) * a.block_size + (g16 - blk * a.block_size)) *
             (size_t)D * C::ELT;
    } else {
      return (size_t)g16 * D * C::ELT;
    }
  };
  const uint8_t* mrow = MASKED ? a.mask + (size_t)b * M : nullptr;

  // 1/sqrt(D) folded with log2(e): p = 2^(s*sl - m*sl).
  const float sl = kLog2e / sqrtf((float)D);

  // Q operand: head h0 + c16, 16-byte chunks (zero for padding heads / d).
  u32x4 qop[C::QCH];
  {
    const bool hv = c16 < gh;
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     ((size_t)b * a.H + h0 + (hv ? c16 : 0)) * (size_t)D * C::ELT;
#pragma unroll
    for (int u = 0; u < C::QCH; ++u) {
      const int d0 = H16 ? (32 * u + 8 * qg) : (16 * u + 4 * qg);
      const bool dv = EXACT || d0 < D;
      qop[u] = sel16(hv && dv, ld16(qp + (size_t)(dv ? d0 : 0) * C::ELT));
    }
  }

  float m_run = kNegInf;
  float l_run = 0.f;  // lane-partial row sum (this lane's keys only)
  f32x4 acc[C::NDB];
#pragma unroll
  for (int i = 0; i < C::NDB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  lds_char* vl = smem + w * C::VBYTES;
  const int klast = k_end - 1;

  struct Chunk {
    u32x4 k[C::NKB][C::QCH];  // K rows in MFMA A-operand layout
    u32x4 v[C::VLOADS];       // V rows, coalesced 16-byte pieces
  };
  // Issue every load of the chunk at `base` (K first, then V).  Addresses
  // are clamped to valid rows.  Nothing here touches the loaded values, so
  // the next chunk's loads stay in flight while the current chunk is
  // computed: rows past the split are zeroed when V is written to LDS or
  // masked to -inf (K), and padded d is zeroed when K feeds the MFMA.
  bool kdv[C::QCH];
#pragma unroll
  for (int u = 0; u < C::QCH; ++u) kdv[u] = EXACT || (H16 ? (32 * u + 8 * qg) : (16 * u + 4 * qg)) < D;
  // Group kb of the chunk at `base` starts at key base + 16 kb; a group
  // wholly past the split is redirected to the split's last group (its rows
  // are masked out later, only the addresses must stay valid).
  const int glast = klast & ~15;
  // The block-table entries of a chunk's groups (paged): scalar loads issued
  // one chunk ahead of the chunk's own loads, so that no load of K or V
  // waits for a table read.
  struct Tab {
    int e[C::NKB];
  };
  auto tab_of = [&](int base) {
    Tab tb;
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      if constexpr (PAGED) {
        tb.e[kb] = btab[min(base + 16 * kb, glast) / a.block_size];
      } else {
        tb.e[kb] = 0;
      }
    }
    return tb;
  };
  auto ldkv = [](const char* p) -> u32x4 {
    if constexpr (NT) {
      return ld16_stream(p);
    } else {
      return ld16(p);
    }
  };
  auto load_chunk = [&](int base, const Tab& tb) {
    Chunk ch;
    int g16[C::NKB];
    size_t goff[C::NKB];
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      g16[kb] = min(base + 16 * kb, glast);
      goff[kb] = group_off(g16[kb], tb.e[kb]);
    }
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      const int key = min(g16[kb] + c16, klast);
      const char* krow = kp + goff[kb] + (size_t)(key - g16[kb]) * D * C::ELT;
#pragma unroll
      for (int u = 0; u < C::QCH; ++u) {
        const int d0 = H16 ? (32 * u + 8 * qg) : (16 * u + 4 * qg);
        if constexpr (EXACT) {
          ch.k[kb][u] = ldkv(krow + (size_t)d0 * C::ELT);
        } else {
          const bool dv = d0 < D;
          ch.k[kb][u] = ldkv(krow + (size_t)(dv ? d0 : 0) * C::ELT);  // zeroed at use
        }
      }
    }
    // one V load instruction covers 64 / CPR (<= 16) rows of one group
#pragma unroll
    for (int it = 0; it < C::VLOADS; ++it) {
      constexpr int RPI = 64 / C::CPR;
      const int grp = (it * RPI) / 16;
      const int piece = it * 64 + lane;
      const int row = piece / C::CPR;
      const int chunk = piece - row * C::CPR;
      const int key = base + row;
      const int d0 = chunk * (16 / C::ELT);
      const bool ok = key < k_end && (EXACT || d0 < D);
      const size_t roff = goff[grp] + (size_t)(min(key, klast) - g16[grp]) * D * C::ELT;
      ch.v[it] = ldkv(vp + roff + (size_t)(ok ? d0 : 0) * C::ELT);  // zeroed at use
    }
    return ch;
  };

  // The workgroup walks its keys in rounds of kstride, wave w taking chunk w
  // of each round.  With a.rotate the walk starts at a round that depends
  // on the unit and split and wraps around, so concurrent workgroups whose
  // ranges start at equally aligned addresses (caches of 8 MB or more per
  // KV head) are not at the same low address bits at the same time; the
  // order is fixed per workgroup, so results stay reproducible.
  const int kstride = kWaves * C::KC;
  const int nround = (k_end - k_begin + kstride - 1) / kstride;
  const int r0 = (a.rotate && nround > 0)
                     ? (int)(((unsigned)unit * 37u + (unsigned)s * 7u) % (unsigned)nround)
                     : 0;
  auto base_of = [&](int t) {
    int r = t + r0;
    if (r >= nround) r -= nround;
    return k_begin + r * kstride + w * C::KC;
  };
  // One chunk of keys: S, softmax, O += V^T P^T (the chunk's loads were
  // issued earlier).
  auto compute = [&](const Chunk& cur, const int base) {
    const auto& kop = cur.k;
    const auto& vreg = cur.v;
    // ---- S^T = K Q^T ------------------------------------------------------
    f32x4 sc[C::NKB];
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < C::QCH; ++u) {
        if constexpr (H16) {
          c = mma16<ET>(EXACT ? kop[kb][u] : sel16(kdv[u], kop[kb][u]), qop[u], c);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            c = mfma_f32(EXACT || kdv[u] ? __uint_as_float(kop[kb][u][e]) : 0.f,
                         __uint_as_float(qop[u][e]), c);
        }
      }
      sc[kb] = c;
    }
    // ---- V chunk to LDS ---------------------------------------------------
#pragma unroll
    for (int it = 0; it < C::VLOADS; ++it) {
      const int piece = it * 64 + lane;
      const int row = piece / C::CPR;
      const int chunk = piece - row * C::CPR;
      const bool ok = base + row < k_end && (EXACT || chunk * (16 / C::ELT) < D);
      lds_st16(vl, v_off<H16, DP>(row, chunk), sel16(ok, vreg[it]));
    }
    // ---- visibility + online softmax --------------------------------------
    float mloc = kNegInf;
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = base + 16 * kb + 4 * qg + r;
        bool vis = key < k_end;
        if constexpr (MASKED) vis = vis && (mrow[min(key, klast)] != 0);
        const float x = vis ? sc[kb][r] : kNegInf;
        sc[kb][r] = x;
        mloc = fmaxf(mloc, x);
      }
    }
    mloc = rows_max(mloc);
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float msl = m_use * sl;
    const float alpha = exp2_hw(m_run * sl - msl);
    m_run = m_new;
    float p[C::NKB][4];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[kb][r] = exp2_hw(fmaf(sc[kb][r], sl, -msl));
        psum += p[kb][r];
      }
    }
    l_run = fmaf(l_run, alpha, psum);
#pragma unroll
    for (int i = 0; i < C::NDB; ++i) acc[i] *= alpha;

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- O^T += V^T P^T ---------------------------------------------------
    if constexpr (H16) {
#pragma unroll
      for (int c = 0; c < C::NKB / 2; ++c) {
        float pp[8] = {p[2 * c][0], p[2 * c][1], p[2 * c][2], p[2 * c][3],
                       p[2 * c + 1][0], p[2 * c + 1][1], p[2 * c + 1][2], p[2 * c + 1][3]};
        const u32x4 bop = pack16x8<ET>(pp);
        const int row_a = 32 * c + 4 * qg + (c16 >> 2);
        const int row_b = row_a + 16;
        const int within = (c16 & 1) << 3;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          const int chunk = 2 * db + ((c16 & 3) >> 1);
          const i16x4 ta = lds_ld_tr16(vl, v_off<H16, DP>(row_a, chunk) + within);
          const i16x4 tb = lds_ld_tr16(vl, v_off<H16, DP>(row_b, chunk) + within);
          acc[db] = mma16<ET>(concat16(ta, tb), bop, acc[db]);
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * kb + 4 * qg + r;
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const float vv = lds_ldf(vl, row * C::ROWB + (16 * db + c16) * 4);
            acc[db] = mfma_f32(vv, p[kb][r], acc[db]);
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  if constexpr (C::PREFETCH) {
    // Two chunk buffers used in turn: the next chunk's loads are in flight
    // while this one is computed.  No chunk is ever copied from one buffer
    // to the other, and inside the loop every load is unconditional, so the
    // compiler's load counters stay exact: a copy, or a load issued on one
    // path only, would make it wait for the chunk in flight as well.
    // The scheduling barriers keep the compiler from sinking a chunk's
    // loads below the previous chunk's math (it does, to save registers).
    Chunk ca, cb;
    Tab ta, tb;  // tables of the next chunk to load into ca / cb
    auto tab_at = [&](int t) { return tab_of(base_of(min(t, nround - 1))); };
    int t = 0;
    if (nround > 0) {
      ta = tab_at(0);
      ca = load_chunk(base_of(0), ta);
      tb = tab_at(1);
    }
    for (; t + 2 < nround; t += 2) {
      cb = load_chunk(base_of(t + 1), tb);
      ta = tab_at(t + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(ca, base_of(t));
      ca = load_chunk(base_of(t + 2), ta);
      tb = tab_at(t + 3);
      __builtin_amdgcn_sched_barrier(0);
      compute(cb, base_of(t + 1));
    }
    if (t + 1 < nround) {
      cb = load_chunk(base_of(t + 1), tb);
      __builtin_amdgcn_sched_barrier(0);
      compute(ca, base_of(t));
      compute(cb, base_of(t + 1));
    } else if (t < nround) {
      compute(ca, base_of(t));
    }
  } else {
    for (int t = 0; t < nround; ++t) {
      const int b0 = base_of(t);
      compute(load_chunk(b0, tab_of(b0)), b0);
    }
  }

  // ---- merge the waves through LDS -----------------------------------
  const float l_tot = rows_sum(l_run);
  __syncthreads();  // all waves are done with their V areas
#if GQA_DECODE_TRACE
  tr_keys = (unsigned long long)wall_clock64();
#endif
  float* cacc = reinterpret_cast<float*>(smem_raw);              // [4][16][DP]
  float* cm = cacc + kWaves * 16 * DP;                           // [4][16]
  float* cl = cm + kWaves * 16;                                  // [4][16]
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    float* dst = cacc + (w * 16 + c16) * DP + 16 * db + 4 * qg;
    *reinterpret_cast<f32x4*>(dst) = acc[db];
  }
  if (qg == 0) {
    cm[w * 16 + c16] = m_run;
    cl[w * 16 + c16] = l_tot;
  }
  __syncthreads();

  // Each thread combines the four waves for quads (head, 4 consecutive d).
  const int DQ = D >> 2;  // D % 4 == 0 for every supported type
  const int nq = gh * DQ;
  const bool single = (S == 1);
  const __amdgpu_buffer_rsrc_t prs = raw_rsrc(
      single ? a.out : a.partials + (size_t)__builtin_amdgcn_readfirstlane(pc.first) * 16 * (D + 4),
      single ? 0u : part_row(S, 0, D));
  for (int q = tid; q < nq; q += kThreads) {
    const int hh = q / DQ;
    const int d = 4 * (q - hh * DQ);
    float mx = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) mx = fmaxf(mx, cm[ww * 16 + hh]);
    const float mu = (mx == kNegInf) ? 0.f : mx;
    float L = 0.f;
    f32x4 A = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = exp2_hw((cm[ww * 16 + hh] - mu) * sl);
      L = fmaf(cl[ww * 16 + hh], f, L);
      const f32x4 c = *reinterpret_cast<const f32x4*>(cacc + (ww * 16 + hh) * DP + d);
#pragma unroll
      for (int e = 0; e < 4; ++e) A[e] = fmaf(c[e], f, A[e]);
    }
    if (single) {
      store_out4<ET, OUTF32>(a.out, ((size_t)b * a.H + h0 + hh) * D + d, A / L);
    } else {
      const uint32_t ro = part_row(s, hh, D);
      st_dev4(prs, ro + 16 + 4 * d, A);
      if (d == 0) st_dev2(prs, ro, f32x2{mx, L});
    }
  }
  if (single) {
#if GQA_DECODE_TRACE
    trace_out(0);
#endif
    return;
  }

  // ---- the last split of the unit to arrive merges all of them -----------
  // Partials are stored and loaded with device-scope accesses, which bypass
  // the non-coherent parts of the per-XCD L2s, so no L2 write-back or
  // invalidation is needed: each wave waits until its stores are complete
  // before the workgroup takes its ticket, and the last workgroup loads the
  // partials only after its ticket shows every split has arrived.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __shared__ int s_last;
  __syncthreads();
  if (tid == 0) {
    const unsigned t = __hip_atomic_fetch_add(a.counters + unit, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    s_last = (t == (unsigned)S - 1u);
  }
  __syncthreads();
#if GQA_DECODE_TRACE
  tr_ticket = (unsigned long long)wall_clock64();
  if (!s_last) trace_out(0);
#endif
  if (!s_last) return;
  if (tid == 0) st_dev(a.counters + unit, 0u);  // ready for the next call
  if (S <= 2) {
    merge_quads<ET, OUTF32, 4, 2>(a, prs, S, b, h0, gh, tid);
  } else if (S <= 4) {
    merge_quads<ET, OUTF32, 2, 4>(a, prs, S, b, h0, gh, tid);
  } else {
    merge_quads<ET, OUTF32, 1, 8>(a, prs, S, b, h0, gh, tid);
  }
#if GQA_DECODE_TRACE
  trace_out(1);
#endif
}

template <int ET, int DP, bool EXACT, bool OUTF32, bool NT>
hipError_t launch_nt(const DecodeArgs& a, hipStream_t stream) {
  const int units = a.B * a.H_kv * a.head_chunks;
  const dim3 grid = a.pieces > 0 ? dim3(a.pieces) : fold_grid(units, (unsigned)a.splits);
  if (a.block_table) {  // the paged form takes no mask
    hipLaunchKernelGGL((decode_kernel<ET, DP, EXACT, false, true, OUTF32, NT>), grid, dim3(kThreads), 0, stream, a);
  } else if (a.mask) {
    hipLaunchKernelGGL((decode_kernel<ET, DP, EXACT, true, false, OUTF32, NT>), grid, dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_kernel<ET, DP, EXACT, false, false, OUTF32, NT>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

// Non-temporal K/V loads unless the group's head chunks re-read the rows
// (fp32 inputs always take them: one kernel instance less per shape, and the
// hint only changes the speed).
template <int ET, int DP, bool EXACT, bool OUTF32>
hipError_t launch_dp(const DecodeArgs& a, hipStream_t stream) {
  if constexpr (ET != kF32) {
    if (a.head_chunks > 1) return launch_nt<ET, DP, EXACT, OUTF32, false>(a, stream);
  }
  return launch_nt<ET, DP, EXACT, OUTF32, true>(a, stream);
}

template <int ET, int DP, bool OUTF32>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  return a.D == DP ? launch_dp<ET, DP, true, OUTF32>(a, stream)
                   : launch_dp<ET, DP, false, OUTF32>(a, stream);
}

template <int ET, bool OUTF32>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  if constexpr (ET == kF32) {
    if (a.D <= 16) return launch_d<ET, 16, OUTF32>(a, stream);
  }
  if (a.D <= 32) return launch_d<ET, 32, OUTF32>(a, stream);
  if (a.D <= 64) return launch_d<ET, 64, OUTF32>(a, stream);
  if (a.D <= 128) return launch_d<ET, 128, OUTF32>(a, stream);
  return launch_d<ET, 256, OUTF32>(a, stream);
}

}  // namespace

DecodePlan plan_decode(int B, int H, int H_kv, int M, int D, bool paged) {
  DecodePlan p{};
  const int g = H / H_kv;
  // At most 16 query heads share one matrix-core tile; larger groups are cut
  // into equal chunks, each a unit that re-reads the group's K/V rows.
  const int chunks = (g + 15) / 16;
  p.head_chunk = (g + chunks - 1) / chunks;
  p.head_chunks = (g + p.head_chunk - 1) / p.head_chunk;
  const long kv_units = (long)B * H_kv;
  p.xcd_group = (p.head_chunks > 1 && kv_units % 8 == 0) ? 1 : 0;
  const long units = kv_units * p.head_chunks;
  // With per-sequence lengths the host does not know how long each sequence
  // is; the paged form has its own target so the two can be tuned apart.
  const long target_wgs = paged ? GQA_DECODE_PAGED_TARGET_WGS : GQA_DECODE_TARGET_WGS;
  const long max_splits = (M + kRoundKeys - 1) / kRoundKeys;
  long splits = (target_wgs + units - 1) / units;
  if (splits > max_splits) splits = max_splits;
  if (splits > 65535) splits = 65535;
  if (splits < 1) splits = 1;
  long kps = (M + splits - 1) / splits;
  kps = (kps + kRoundKeys - 1) / kRoundKeys * kRoundKeys;
  splits = (M + kps - 1) / kps;
  p.splits = (int)splits;
  p.keys_per_split = (int)kps;
  if (p.splits > 1) {
    // splits > 1 only when units < target_wgs <= kMaxCounters, so the
    // counters fit their fixed area
    p.partials_bytes = (size_t)units * p.splits * 16 * (size_t)(D + 4) * 4;
    p.workspace_bytes = kCounterBytes + p.partials_bytes;
  }
  const long groups = units * ((M + 63) / 64);  // 64-key groups of the longest batch
  if (paged && GQA_DECODE_PAGED_PIECES && max_splits > 1 && units < kMaxCounters &&
      groups < (1L << 30)) {
    // length-balanced pieces planned on the device (in int arithmetic, hence
    // the bound on the group count), one workgroup per piece: one wave of
    // workgroups for few units, two workgroups per unit for many, a
    // multiple of 8 for the XCD-grouped order
    const long G = units < target_wgs ? target_wgs : (2 * units + 7) / 8 * 8;
    p.pieces = (int)G;
    p.xcd_group = 0;
    p.partials_bytes = (size_t)p.pieces * 16 * (size_t)(D + 4) * 4;
    p.workspace_bytes = kCounterBytes + p.partials_bytes;
  }
  if (GQA_DECODE_WIDE && !paged && g > GQA_DECODE_WIDE_MIN_G) {
    // the prefill view: B * H_kv units of ceil(g / 128) row blocks, two
    // workgroups per CU; splits of a multiple of 64 keys
    const long wunits = kv_units * ((g + 127) / 128);
    long ws = (GQA_DECODE_WIDE_TARGET_WGS + wunits - 1) / wunits;
    const long wmax = (M + 63) / 64;
    if (ws > wmax) ws = wmax;
    if (ws > 65535) ws = 65535;
    if (ws < 1) ws = 1;
    long wk = (M + ws - 1) / ws;
    wk = (wk + 63) / 64 * 64;
    ws = (M + wk - 1) / wk;
    p.wide = 1;
    p.wide_splits = (int)ws;
    p.wide_kps = (int)wk;
    p.partials_bytes = ws > 1 ? (size_t)B * H * ws * (size_t)(D + 4) * 4 : 0;
    p.workspace_bytes = ws > 1 ? kCounterBytes + p.partials_bytes : 0;
  }
  return p;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  switch (a.in_type) {
    case kBF16:
      return a.out_f32 ? launch_t<kBF16, true>(a, stream) : launch_t<kBF16, false>(a, stream);
    case kF16:
      return a.out_f32 ? launch_t<kF16, true>(a, stream) : launch_t<kF16, false>(a, stream);
    default:
      return launch_t<kF32, true>(a, stream);
  }
}

}  // namespace gqa
