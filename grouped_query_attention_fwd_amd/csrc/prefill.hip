// Prefill (N query positions) grouped-query attention forward for gfx950.
//
// Operation: for each batch row b, query head h and position i,
//   o[b,h,i,:] = softmax_{j visible}(q[b,h,i,:] . k[b,h/g,j,:] / sqrt(D)) v[b,h/g,j,:]
// ("28. Grouped-Query Attention (GQA)", *Reference solution*: repeat-
// interleave grouping, 1/sqrt(D) scale, [B,N,M] mask broadcast over heads;
// "Grouped-Query Attention Explained Simply", *Minimal implementation*: the
// causal self-attention mask, read as key j visible to query i iff j <= i),
// generalised to a band: key j is visible to query i iff it lies within
// window_left keys before and window_right keys after position i + q_offset
// (either side may be unbounded); causal is the band with right edge 0.
//
// Design (flash-style, dense contraction on the matrix cores):
//   * A workgroup of four waves (eight for 16-bit 256-wide rows) takes the
//     query heads of one KV group that
//     share a block of positions (HG heads x PB positions, HG in {4,2,1});
//     the K/V tiles it streams are therefore read once for all of its heads
//     (the zero head stride of "Multi-Query Attention", *Implementation*) and
//     all heads share one band / mask frontier.
//   * K and V tiles of BN keys are double-buffered in LDS, as four distinct
//     LDS objects with the tile loop unrolled by two (every access names its
//     stage).  16-bit tiles whose rows need no column padding go straight
//     from global memory to LDS (no staging registers): whole tiles with
//     buffer_load_dwordx4 ... lds from a descriptor, a scalar row offset and
//     a loop-invariant lane offset (no vector instructions), a ragged last
//     tile with global_load_lds_dwordx4 on clamped rows.  The XOR swizzle of
//     the LDS rows is applied by permuting each lane's global source.  Other
//     cases stage through registers.  The next tile's copy is issued before
//     the current tile's math.
//   * Each wave owns 16*QB query rows.  S^T = K Q^T and O^T = V^T P^T run on
//     v_mfma_f32_16x16x32_bf16 / _f16 (16-bit inputs) or
//     v_mfma_f32_16x16x4f32 (fp32 inputs); V^T is read with the transposing
//     ds_read_b64_tr_b16.  P is rounded to the input type
//     (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32) for the 16-bit product; all
//     accumulation is fp32.
//   * Online softmax per query row with exp2 and a scale of log2(e)/sqrt(D);
//     a lane owns one query row per 16-row block, so its running max and
//     rescale factor never leave the lane.  With 16-bit inputs the row sums
//     of the rounded weights are one more MFMA against an all-ones operand.
//   * Band (causal is the band with right edge 0): each workgroup and wave
//     derive their key range from it, tiles outside it are never visited,
//     and only tiles that cross a band edge, the end of the keys or a mask
//     pay for per-element visibility.  Mask: tiles with no visible pair are
//     skipped entirely (no K/V copy, no MFMA), decided by a workgroup vote.
//   * Dispatch: workgroup L runs on XCD L % 8; each XCD walks its own units
//     one after another (all position blocks of a unit together, heaviest
//     causal blocks first), so the tiles in flight on an XCD stay in its L2.
//   * Optional key splits (used by the decode of large groups, whose heads
//     are the query rows here): workgroup column s covers one key range and
//     writes a partial (m, l, acc) per row.  With 16-row waves the splits of
//     a position block merge the partials themselves, each a slice of the
//     rows, after the last one has arrived (no second launch); otherwise a
//     small kernel merges them.
#include <atomic>

#include "gqa_device.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

// Waves per workgroup (4 or 8).  With 8 waves the bf16 tiles hold 128 keys,
// so each barrier and each tile copy is amortised over twice the math.
#ifndef GQA_PREFILL_WAVES
#define GQA_PREFILL_WAVES 4
#endif
constexpr int kWaves = GQA_PREFILL_WAVES;
constexpr int kThreads = 64 * kWaves;
#ifndef GQA_PREFILL_SETPRIO
#define GQA_PREFILL_SETPRIO 0
#endif
#ifndef GQA_PREFILL_SGB
#define GQA_PREFILL_SGB 0
#endif
#ifndef GQA_PREFILL_XCD_MAJOR
#define GQA_PREFILL_XCD_MAJOR 1
#endif
// 1: causal blocks of very unequal weight use order 2 (below).  Measured
// 0.6-1.5 % faster on the causal N = 4096 prefill but with twice the HBM
// fetch (four units in flight per XCD overflow its L2), so off.
#ifndef GQA_PREFILL_XCD_LPT
#define GQA_PREFILL_XCD_LPT 0
#endif
// Rescale threshold of the online softmax, in log2 units (weights <= 2^8).
constexpr float kLazy = 8.f;

// QBO > 0 sets the 16-row query blocks per wave (the decode of large groups
// uses 1: its 64 heads fill all four waves of one block).
template <bool H16, int DP, int QBO = 0>
struct PreCfg {
  static constexpr int ELT = H16 ? 2 : 4;
#ifndef GQA_PREFILL_QB
#define GQA_PREFILL_QB 2
#endif
  static constexpr int QB = QBO > 0 ? QBO : ((H16 && DP <= 128) ? GQA_PREFILL_QB : 1);  // 16-row query blocks per wave
  static constexpr int RW = 16 * QB;                       // query rows per wave
#ifndef GQA_PREFILL_BN
#define GQA_PREFILL_BN 64
#endif
// 16-bit tiles of 256-wide rows: 32 keys, so that two workgroups fit a CU
// (64 KB of LDS and at most 256 registers each; with 64 keys a workgroup
// takes 128 KB of LDS and 320-380 registers, one per CU).
#ifndef GQA_PREFILL_BN256
#define GQA_PREFILL_BN256 32
#endif
  static constexpr int BN = H16 ? (DP == 256 ? GQA_PREFILL_BN256 : GQA_PREFILL_BN)
                                 : (DP <= 64 ? 64 : (DP == 128 ? 32 : 16));  // keys per tile
  static constexpr int NKB = BN / 16;
  static constexpr int NDB = DP / 16;
  static constexpr int QCH = H16 ? DP / 32 : DP / 16;     // 16-byte operand chunks per lane
  static constexpr int CPR = DP * ELT / 16;                // 16-byte chunks per row
  static constexpr int ROWB = H16 ? DP * 2 : DP * 4 + 16; // LDS row stride
  static constexpr int TILE = BN * ROWB;                   // bytes of one K or V tile
  static constexpr int STAGE = 2 * TILE;                   // K + V
  static constexpr int PIECES = 2 * BN * CPR;              // 16-byte pieces per stage
#ifndef GQA_PREFILL_WAVES256
#define GQA_PREFILL_WAVES256 8
#endif
  // waves per workgroup: 16-bit tiles of 256-wide rows share each K/V tile
  // among eight waves (3.5 % faster on the causal D = 256 prefill than four)
  static constexpr int NW = (H16 && DP == 256) ? GQA_PREFILL_WAVES256 : kWaves;
  static constexpr int THREADS = 64 * NW;
  static constexpr int PPT = PIECES / THREADS;             // pieces per thread
  static constexpr int KSWZ = (CPR < 16 ? CPR : 16) - 1;   // K row swizzle mask
  static constexpr int SPR = DP / 16;                      // 32-byte segments per 16-bit row
  static constexpr int VSWZ = (SPR < 8 ? SPR : 8) - 1;     // V row swizzle mask
  // direct copies: one wave instruction fills 1 KB = RPI rows of a tile
  static constexpr int RPI = H16 ? 1024 / ROWB : 1;
  static constexpr int DMA_INSTS = H16 ? BN / RPI : 0;                  // per K or V tile
  static constexpr int DMA_PER_TILE = (DMA_INSTS + NW - 1) / NW;  // per wave
  static_assert(PIECES % THREADS == 0, "stage must split evenly over the threads");
  static_assert(!H16 || BN % 32 == 0, "16-bit P.V works on whole 32-key halves of a tile");
  static_assert(!H16 || (BN % RPI == 0), "direct copy must cover whole rows");
};

// Direct global -> LDS copy of 16 bytes per lane through a buffer
// descriptor (buffer_load_dwordx4 ... lds): the source of a lane is the
// descriptor's base + `soff` (wave-uniform, a scalar register) + `voff`
// (per lane); the LDS destination is `lds_base` + 16 * lane.  Callers keep
// every source inside the descriptor's range.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                          lds_char* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16,
                                           voff, soff, 0, 0);
}

template <bool H16, int DP>
__device__ __forceinline__ uint32_t k_off(int row, int chunk) {
  using C = PreCfg<H16, DP>;
  if constexpr (H16) return row * C::ROWB + ((chunk ^ (row & C::KSWZ)) << 4);
  else return row * C::ROWB + (chunk << 4);
}

template <bool H16, int DP>
__device__ __forceinline__ uint32_t v_off(int row, int chunk) {
  using C = PreCfg<H16, DP>;
  if constexpr (H16) return row * C::ROWB + ((chunk ^ (2 * (row & C::VSWZ))) << 4);
  else return row * C::ROWB + (chunk << 4);
}

// Bound on the polls of a workgroup that waits for the other key splits of
// its position block (each poll is a device-scope load, at least about
// half a microsecond): in a normal launch they all arrive within
// microseconds; the bound only keeps the wait finite if they could not run
// at the same time.
constexpr int kMergeSpin = 1 << 16;

// Merge rows [r0, r1) of one position block's key-split partials (`prs`:
// rows x S splits x [m, l, -, -, acc[0..D)] fp32, read with device-scope
// loads) into output rows orow0 + r, by `nt` threads (this one is `t`), four
// elements of one row per item.  Splits are combined in split order, NB per
// memory round trip (indexes clamped to the last split): a running m*, with
// o = sum_s acc_s 2^((m_s - m*) sl) / sum_s l_s 2^((m_s - m*) sl).
template <int ET, bool OUTF32, int NB>
__device__ __forceinline__ void merge_rows_nb(const PrefillArgs& a, __amdgpu_buffer_rsrc_t prs,
                                              size_t orow0, int r0, int r1, int S, int D, int t,
                                              int nt) {
  const float sl = kLog2e / sqrtf((float)D);
  const int DQ = D >> 2;  // D % 4 == 0 for every supported type
  const uint32_t sbytes = (uint32_t)(D + 4) * 4u;
  const int n = (r1 - r0) * DQ;
  for (int it = t; it < n; it += nt) {
    const int rr = it / DQ;
    const int d = 4 * (it - rr * DQ);
    const int r = r0 + rr;
    const uint32_t base = (uint32_t)r * (uint32_t)S * sbytes;
    float mx = kNegInf, ls = 0.f;
    f32x4 A = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += NB) {
      f32x2 ml[NB];
      f32x4 pa[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const uint32_t o = base + (uint32_t)min(s0 + u, S - 1) * sbytes;
        ml[u] = ld_dev2(prs, o);
        pa[u] = ld_dev4(prs, o + 16u + 4u * d);
      }
      float cm = kNegInf;
#pragma unroll
      for (int u = 0; u < NB; ++u)
        if (s0 + u < S) cm = fmaxf(cm, ml[u][0]);
      const float nm = fmaxf(mx, cm);
      if (nm == kNegInf) continue;  // nothing visible yet
      const float f0 = (mx == kNegInf) ? 0.f : exp2_hw((mx - nm) * sl);
      ls *= f0;
#pragma unroll
      for (int e = 0; e < 4; ++e) A[e] *= f0;
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        if (s0 + u < S) {
          const float f = exp2_hw((ml[u][0] - nm) * sl);
          ls = fmaf(ml[u][1], f, ls);
#pragma unroll
          for (int e = 0; e < 4; ++e) A[e] = fmaf(pa[u][e], f, A[e]);
        }
      }
      mx = nm;
    }
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = A[e] / ls;
    const size_t oi = (orow0 + r) * (size_t)D + d;
    if constexpr (OUTF32) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + oi) = o;
    } else {
      u32x2 pk = {pack16<ET>(o[0], o[1]), pack16<ET>(o[2], o[3])};
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + oi) = pk;
    }
  }
}

// Up to 16 splits in one round trip, more eight at a time.
template <int ET, bool OUTF32>
__device__ __forceinline__ void merge_block_rows(const PrefillArgs& a, __amdgpu_buffer_rsrc_t prs,
                                                 size_t orow0, int r0, int r1, int S, int D, int t,
                                                 int nt) {
  if (S <= 16) merge_rows_nb<ET, OUTF32, 16>(a, prs, orow0, r0, r1, S, D, t, nt);
  else merge_rows_nb<ET, OUTF32, 8>(a, prs, orow0, r0, r1, S, D, t, nt);
}

// ET: element type of q, k, v.  DIRECT: 16-bit elements with D == DP, tiles
// copied straight into LDS.  MASKED: a [B,N,M] mask is given.
template <int ET, int DP, bool DIRECT, bool MASKED, bool OUTF32, int QBO>
__global__ void __launch_bounds__((PreCfg<ET != kF32, DP, QBO>::THREADS),
                                  (8 / PreCfg<ET != kF32, DP, QBO>::NW))
    prefill_kernel(PrefillArgs a, int HG, int units, int npb, int order) {
  constexpr bool H16 = ET != kF32;  // 16-bit elements: bf16 or fp16
  using C = PreCfg<H16, DP, QBO>;
  static_assert(!DIRECT || H16, "direct copies are for 16-bit tiles");
  // Two stages as two distinct LDS objects: with the loop unrolled by two
  // every access names its stage statically, so the compiler can tell that
  // reads of one stage never alias the copy in flight into the other (it
  // would otherwise wait for that copy before each transposing V read).
  __shared__ __attribute__((aligned(16))) char k0_raw[C::TILE];
  __shared__ __attribute__((aligned(16))) char v0_raw[C::TILE];
  __shared__ __attribute__((aligned(16))) char k1_raw[C::TILE];
  __shared__ __attribute__((aligned(16))) char v1_raw[C::TILE];
  lds_char* const k0s = (lds_char*)k0_raw;
  lds_char* const v0s = (lds_char*)v0_raw;
  lds_char* const k1s = (lds_char*)k1_raw;
  lds_char* const v1s = (lds_char*)v1_raw;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int lane = tid & 63;
  const int c16 = lane & 15;
  const int qg = lane >> 4;

  const int D = DIRECT ? DP : a.D;
  const int N = a.N, M = a.M;
  const int groups_per_kv = a.g / HG;
  // Workgroup -> (unit, position block).  Workgroups are dispatched to the
  // 8 XCDs round-robin (L % 8).  With order 1 each XCD walks its own units
  // one after another (all blocks of a unit, heaviest first), so the K/V
  // tiles in flight on an XCD come from about one unit and stay in its L2.
  // Order 2 is for blocks of very unequal weight (causal with N close to
  // M): each XCD runs its units side by side, heaviest blocks of all of them
  // first, so the light blocks fill the end (longest-processing-time first).
  const int L = (int)(blockIdx.x + gridDim.x * blockIdx.z);
  if (L >= units * npb) return;  // the end of a folded grid (workgroup-uniform)
  int unit, pbi;
  if (order) {
    const int x = L & 7;
    const int i = L >> 3;
    int lu;
    if (order == 2) {
      // the XCD's units side by side, all their heaviest blocks first
      const int upx = units >> 3;
      pbi = i / upx;
      lu = i - pbi * upx;
    } else {
      lu = i / npb;
      pbi = i - lu * npb;
    }
    unit = lu * 8 + x;
  } else {
    unit = L % units;
    pbi = L / units;
  }
  // the band's upper edge makes later blocks heavier: run them first
  const int pblk = (a.wr >= 0 && a.wl < 0) ? (npb - 1 - pbi) : pbi;
  const int b = unit / (a.H_kv * groups_per_kv);
  const int rem = unit - b * (a.H_kv * groups_per_kv);
  const int j = rem / groups_per_kv;
  const int hgi = rem - j * groups_per_kv;
  const int wph = C::NW / HG;        // waves per head
  const int PB = wph * C::RW;         // positions per workgroup
  const int p0 = pblk * PB;
  const int h = j * a.g + hgi * HG + (w % HG);
  const int wp0 = p0 + (w / HG) * C::RW;  // this wave's first position

  const size_t kv_base = ((size_t)b * a.H_kv + j) * (size_t)M * D;
  const char* kp = reinterpret_cast<const char*>(a.k) + kv_base * C::ELT;
  const char* vp = reinterpret_cast<const char*>(a.v) + kv_base * C::ELT;
  const uint8_t* mb = MASKED ? a.mask + (size_t)b * a.mask_bs : nullptr;
  const size_t mrs = MASKED ? (size_t)a.mask_rs : 0;   // mask row stride
  const float sl = kLog2e / sqrtf((float)D);

  // Band edges of query position pos, clamped to [0, M]: keys
  // [key_lo(pos), key_hi(pos)) are visible (before any mask).  Both edges
  // grow with pos.
  auto key_lo = [&](int pos) -> int {
    if (a.wl < 0) return 0;
    const long long x = (long long)pos + a.q_offset - a.wl;   // no int overflow
    return (int)(x < 0 ? 0 : (x > M ? M : x));
  };
  auto key_hi = [&](int pos) -> int {
    if (a.wr < 0) return M;
    const long long x = (long long)pos + a.q_offset + a.wr + 1;
    return (int)(x < 0 ? 0 : (x > M ? M : x));
  };
  // key range of the workgroup and of this wave, within this key split
  const int s_lo = (int)blockIdx.y * a.kps;
  const int s_hi = min(M, s_lo + a.kps);
  const int last_pos = min(N, p0 + PB);          // exclusive
  const int kbeg = max(key_lo(p0), s_lo);
  const int kend = (p0 < N) ? min(key_hi(last_pos - 1), s_hi) : 0;
  const int t_first = kbeg / C::BN;
  const int ntiles = (kend + C::BN - 1) / C::BN;
  const int w_last = min(N, wp0 + C::RW);        // exclusive
  const int w_kbeg = max(key_lo(wp0), s_lo);
  const int w_kend = (wp0 >= N) ? 0 : min(key_hi(w_last - 1), s_hi);
  // keys every row of this wave sees: [w_full_lo, w_full_hi)
  const int w_full_lo = (wp0 >= N) ? M : key_lo(w_last - 1);
  const int w_full_hi = (wp0 >= N) ? 0 : key_hi(wp0);

  // Q operands for this wave's rows (zero for rows past N and padded d)
  u32x4 qop[C::QB][C::QCH];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int pos = wp0 + 16 * qb + c16;
    const bool pv = pos < N;
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     (((size_t)b * a.H + h) * N + (pv ? pos : 0)) * (size_t)D * C::ELT;
#pragma unroll
    for (int u = 0; u < C::QCH; ++u) {
      const int d0 = H16 ? (32 * u + 8 * qg) : (16 * u + 4 * qg);
      const bool dv = DIRECT || d0 < D;
      qop[qb][u] = sel16(pv && dv, ld16(qp + (size_t)(dv ? d0 : 0) * C::ELT));
    }
  }

  // nmsl = -m_run * sl, the exponent offset of the weights (0 while the
  // row has seen no visible key); it changes only with the reference.
  float m_run[C::QB], l_run[C::QB], nmsl[C::QB];
  f32x4 acc[C::QB][C::NDB];
  // 16-bit inputs: the row sums of the weights come from the matrix cores
  // (lacc, every register of a lane holds its row's sum), fp32: l_run
  f32x4 lacc[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    m_run[qb] = kNegInf;
    l_run[qb] = 0.f;
    nmsl[qb] = 0.f;
    lacc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < C::NDB; ++i) acc[qb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Workgroup vote: does tile t hold any visible (position, key) pair?
  auto tile_visible = [&](int t) -> bool {
    int any = 0;
    const int k0 = t * C::BN;
    for (int idx = tid; idx < PB * C::BN; idx += C::THREADS) {
      const int i = idx / C::BN;
      const int key = k0 + (idx - i * C::BN);
      const int pos = p0 + i;
      if (pos < N && key < kend && key >= key_lo(pos) && key < key_hi(pos) &&
          mb[(size_t)pos * mrs + key])
        any = 1;
    }
    return __syncthreads_or(any) != 0;
  };
  auto next_tile = [&](int t) -> int {
    if constexpr (MASKED) {
      while (t < ntiles && !tile_visible(t)) ++t;
    }
    return t;
  };

  // ---- tile copies -----------------------------------------------------------
  u32x4 stage[DIRECT ? 1 : C::PPT];
  // DIRECT copies: global -> LDS, no registers.  which = 0: K, 1: V.
  // A tile that lies wholly inside the keys needs no clamping: its source is
  // a buffer descriptor over this (b, KV head)'s rows, a wave-uniform row
  // offset (scalar register) and a per-lane offset that does not change from
  // tile to tile (the swizzle depends only on the row's low bits, which the
  // advance of C::NW * RPI rows per instruction leaves alone for D <= 128),
  // so such a copy costs no vector instructions.  Slabs of 2^31 bytes or
  // more take the clamped path below.
  constexpr bool kDmaInvariant = DIRECT && ((C::NW * C::RPI) % (C::KSWZ + 1) == 0) &&
                                 ((C::NW * C::RPI) % (C::VSWZ + 1) == 0);
  const bool dma_buf = kDmaInvariant && (long long)M * C::ROWB <= 0x7fffffffLL;
  uint32_t dma_off[2] = {0u, 0u};
  __amdgpu_buffer_rsrc_t dma_rsrc[2];
  if constexpr (kDmaInvariant) {
    const int lrow = lane / C::CPR;
    const int slot = lane - lrow * C::CPR;
    const int row0 = w * C::RPI + lrow;
    dma_off[0] = (uint32_t)(row0 * C::ROWB + ((slot ^ (row0 & C::KSWZ)) << 4));
    dma_off[1] = (uint32_t)(row0 * C::ROWB + ((slot ^ (2 * (row0 & C::VSWZ))) << 4));
    const uint32_t slab = dma_buf ? (uint32_t)M * C::ROWB : 0u;
    dma_rsrc[0] = raw_rsrc(kp, slab);
    dma_rsrc[1] = raw_rsrc(vp, slab);
  }
  auto dma_half = [&](int t, lds_char* dst_tile, int which) {
    const int k0 = t * C::BN;
    const char* src = which ? vp : kp;
    const int lrow = lane / C::CPR;            // row within the instruction's 1 KB
    const int slot = lane - lrow * C::CPR;     // LDS chunk slot of this lane
#pragma unroll
    for (int i = 0; i < C::DMA_PER_TILE; ++i) {
      if (C::DMA_INSTS % C::NW != 0 && i * C::NW + w >= C::DMA_INSTS) break;  // wave-uniform
      const int row = (i * C::NW + w) * C::RPI + lrow;
      const int key = min(k0 + row, M - 1);
      // the chunk that belongs at `slot` under this row's swizzle
      const int chunk = which ? (slot ^ (2 * (row & C::VSWZ))) : (slot ^ (row & C::KSWZ));
      dma16(src + ((size_t)key * DP + chunk * 8) * 2, dst_tile + (i * C::NW + w) * 1024);
    }
  };
  auto dma_tile = [&](int t, lds_char* kdst, lds_char* vdst) {
    const int k0 = t * C::BN;
    if constexpr (kDmaInvariant) {
      if (__builtin_expect(dma_buf && k0 + C::BN <= M, 1)) {
#pragma unroll
        for (int which = 0; which < 2; ++which) {
#pragma unroll
          for (int i = 0; i < C::DMA_PER_TILE; ++i) {
            if (C::DMA_INSTS % C::NW != 0 && i * C::NW + w >= C::DMA_INSTS) break;
            dma16_buf(dma_rsrc[which], dma_off[which],
                      (uint32_t)(k0 + i * C::NW * C::RPI) * C::ROWB,
                      (which ? vdst : kdst) + (i * C::NW + w) * 1024);
          }
        }
        return;
      }
    }
    dma_half(t, kdst, 0);
    dma_half(t, vdst, 1);
  };
  auto load_stage = [&](int t) {          // staged: global -> registers
    const int k0 = t * C::BN;
#pragma unroll
    for (int it = 0; it < C::PPT; ++it) {
      const int piece = it * C::THREADS + tid;
      const int which = piece / (C::BN * C::CPR);      // 0 = K, 1 = V
      const int rr = piece - which * (C::BN * C::CPR);
      const int row = rr / C::CPR;
      const int chunk = rr - row * C::CPR;
      const int key = k0 + row;
      const int d0 = chunk * (16 / C::ELT);
      const char* src = which ? vp : kp;
      const bool ok = key < M && d0 < D;
      stage[it] = sel16(ok, ld16(src + ((size_t)min(key, M - 1) * D + (ok ? d0 : 0)) * C::ELT));
    }
  };
  auto store_stage = [&](lds_char* kt, lds_char* vt) {  // staged: registers -> LDS
#pragma unroll
    for (int it = 0; it < C::PPT; ++it) {
      const int piece = it * C::THREADS + tid;
      const int which = piece / (C::BN * C::CPR);
      const int rr = piece - which * (C::BN * C::CPR);
      const int row = rr / C::CPR;
      const int chunk = rr - row * C::CPR;
      if (which) lds_st16(vt, v_off<H16, DP>(row, chunk), stage[it]);
      else lds_st16(kt, k_off<H16, DP>(row, chunk), stage[it]);
    }
  };

  // ---- per-tile building blocks ------------------------------------------
  typedef f32x4 Scores[C::QB][C::NKB];

  // S^T = K Q^T for the tile in K buffer `kbuf_lds`.
  auto tile_scores = [&](const lds_char* kbuf_lds, Scores& sc) {
    if constexpr (GQA_PREFILL_SETPRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) sc[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (H16 && DIRECT) {
      // D-chunk outermost: each step reads one K chunk per key block and
      // issues NKB * QB independent MFMAs, so no accumulator chain waits on
      // its own previous MFMA (measured 1 % faster than key block outermost;
      // the staged-copy kernels keep the other order, which needs fewer
      // registers).  The next step's K chunk is read before this step's
      // MFMAs (two operand sets in turn), so its LDS latency runs under them.
      u32x4 kop[2][C::NKB];
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
        kop[0][kb] = lds_ld16(kbuf_lds, k_off<H16, DP>(16 * kb + c16, qg));
#pragma unroll
      for (int u = 0; u < C::QCH; ++u) {
        if (u + 1 < C::QCH) {
#pragma unroll
          for (int kb = 0; kb < C::NKB; ++kb)
            kop[(u + 1) & 1][kb] = lds_ld16(kbuf_lds, k_off<H16, DP>(16 * kb + c16, 4 * (u + 1) + qg));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb) sc[qb][kb] = mma16<ET>(kop[u & 1][kb], qop[qb][u], sc[qb][kb]);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
        for (int u = 0; u < C::QCH; ++u) {
          const u32x4 kop = lds_ld16(kbuf_lds, k_off<H16, DP>(16 * kb + c16, 4 * u + qg));
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb) {
            if constexpr (H16) {
              sc[qb][kb] = mma16<ET>(kop, qop[qb][u], sc[qb][kb]);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                sc[qb][kb] = mfma_f32(__uint_as_float(kop[e]), __uint_as_float(qop[qb][u][e]), sc[qb][kb]);
            }
          }
        }
      }
    }
    if constexpr (GQA_PREFILL_SETPRIO) __builtin_amdgcn_s_setprio(0);
  };
  // Invisible (position, key) pairs of tile t get -inf; only tiles that
  // cross a band edge, the end of the keys or a mask pay for this.
  auto tile_mask = [&](int t, Scores& sc) {
    const int k0 = t * C::BN;
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      const int pos = wp0 + 16 * qb + c16;
      const int lo = key_lo(pos), hi = key_hi(pos);  // keys in [lo, hi) are in range
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + 16 * kb + 4 * qg + r;
          bool vis = key >= lo && key < hi;
          if constexpr (MASKED) {
            const uint8_t mbyte = mb[(size_t)min(pos, N - 1) * mrs + min(key, M - 1)];
            vis = vis && (mbyte != 0) && (pos < N);
          }
          sc[qb][kb][r] = vis ? sc[qb][kb][r] : kNegInf;
        }
      }
    }
  };
  // Byte offsets of this lane's transposing V reads: row 4 qg + c16 / 4 of
  // the tile (plus a multiple of 16 rows, which keeps the swizzle), 16-byte
  // chunk 2 db + (c16 % 4) / 2, half (c16 % 2).  Loop-invariant.
  uint32_t vt_off[C::NDB];
  if constexpr (H16) {
    const int vr = 4 * qg + (c16 >> 2);
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
      vt_off[db] = v_off<H16, DP>(vr, 2 * db + ((c16 & 3) >> 1)) + ((c16 & 1) << 3);
  }
  // Online softmax and O^T += V^T P^T for one tile.
  // Weights are p = 2^(s*sl - m_ref*sl) against a per-row reference max
  // m_ref (m_run).  The reference, and with it acc and l, only moves when
  // some row of the wave has a score more than kLazy (log2 units) above it,
  // so p <= 2^kLazy and most tiles skip the rescale; softmax does not depend
  // on the reference, so the result is the same.
  // The weights are formed one 32-key half at a time and each half's P.V
  // MFMAs follow it, so the exp work of the second half can overlap the
  // matrix-core work of the first.
  auto tile_softmax_pv = [&](Scores& sc, lds_char* vbuf_lds) {
    // The reference moves only when some row's maximum passes it by more
    // than kLazy (log2 units).  The test is monotone in the score, so asking
    // it of each lane's own maximum gives the same wave-wide answer as asking
    // it of the row maxima; the cross-lane reduction is only needed when the
    // reference moves.
    float mlane[C::QB];
    bool bump = false;
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[qb][kb][r]);
      mlane[qb] = mx;
      bump = bump || ((mx - m_run[qb]) * sl > kLazy);
    }
    if (__builtin_amdgcn_ballot_w64(bump) != 0) {   // wave-uniform, rare
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        const float m_new = fmaxf(m_run[qb], rows_max(mlane[qb]));
        const float alpha = (m_new == kNegInf) ? 1.f : exp2_hw((m_run[qb] - m_new) * sl);
        m_run[qb] = m_new;
        nmsl[qb] = (m_new == kNegInf) ? 0.f : -(m_new * sl);
        l_run[qb] *= alpha;
        lacc[qb] *= alpha;
#pragma unroll
        for (int i = 0; i < C::NDB; ++i) acc[qb][i] *= alpha;
      }
    }
    if constexpr (H16) {
#pragma unroll
      for (int c = 0; c < C::NKB / 2; ++c) {
        // Direct-copy kernels read this half's V operands first, so their
        // LDS latency runs under the exps; with the K read-ahead above this
        // took the waits for LDS reads from 16 to 5 per tile (about 2 %
        // faster).  The staged-copy kernels hold their copy in registers and
        // read V as they go.
        u32x4 vops[DIRECT ? C::NDB : 1];
        if constexpr (DIRECT) {
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const i16x4 ta = lds_ld_tr16(vbuf_lds, vt_off[db] + (32 * c) * C::ROWB);
            const i16x4 tb = lds_ld_tr16(vbuf_lds, vt_off[db] + (32 * c + 16) * C::ROWB);
            vops[db] = concat16(ta, tb);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        u32x4 bop[C::QB];
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb) {
          float pp[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pp[e] = exp2_hw(fmaf(sc[qb][2 * c + (e >> 2)][e & 3], sl, nmsl[qb]));
          bop[qb] = pack16x8<ET>(pp);
        }
        // Row sums on the matrix cores: with an all-ones A operand the
        // product's element (i, row) is the sum of the row's rounded weights
        // over the 32 keys, the same for every i, in the lane that owns the
        // row.  This replaces 32 vector adds per tile and sums exactly the
        // weights the P.V product uses (measured 1.5-2.4 % faster).
        {
          const uint32_t one2 = ET == kBF16 ? 0x3F803F80u : 0x3C003C00u;
          const u32x4 ones = {one2, one2, one2, one2};
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb) lacc[qb] = mma16<ET>(ones, bop[qb], lacc[qb]);
        }
        if constexpr (DIRECT) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int db = 0; db < C::NDB; ++db)
#pragma unroll
            for (int qb = 0; qb < C::QB; ++qb) acc[qb][db] = mma16<ET>(vops[db], bop[qb], acc[qb][db]);
        } else {
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const i16x4 ta = lds_ld_tr16(vbuf_lds, vt_off[db] + (32 * c) * C::ROWB);
            const i16x4 tb = lds_ld_tr16(vbuf_lds, vt_off[db] + (32 * c + 16) * C::ROWB);
            const u32x4 vop = concat16(ta, tb);
#pragma unroll
            for (int qb = 0; qb < C::QB; ++qb) acc[qb][db] = mma16<ET>(vop, bop[qb], acc[qb][db]);
          }
        }
      }
      if constexpr (GQA_PREFILL_SGB && C::NKB == 4 && C::QB == 2) {
        // exp work of the second key half interleaved with the first half's MFMAs
        constexpr int kMf = C::NDB * C::QB;   // MFMAs per half
        __builtin_amdgcn_sched_group_barrier(0x002, 40, 0);
#pragma unroll
        for (int i = 0; i < kMf; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
#pragma unroll
        for (int i = 0; i < kMf; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
        float pf[C::QB][4];
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pf[qb][r] = exp2_hw(fmaf(sc[qb][kb][r], sl, nmsl[qb]));
            l_run[qb] += pf[qb][r];
          }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * kb + 4 * qg + r;
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const float vv = lds_ldf(vbuf_lds, row * C::ROWB + (16 * db + c16) * 4);
#pragma unroll
            for (int qb = 0; qb < C::QB; ++qb) acc[qb][db] = mfma_f32(vv, pf[qb][r], acc[qb][db]);
          }
        }
      }
    }
  };
  auto tile_needs_mask = [&](int t) {
    const int k0 = t * C::BN;
    return MASKED || (k0 + C::BN > M) || k0 < w_full_lo || k0 + C::BN > w_full_hi;
  };

  // Double-buffered tile loop: the copy of the next visible tile into the
  // other stage is issued before this tile's math (direct copies need no
  // registers; staged copies land in registers and are written to LDS after
  // the math).  A stage holds the K tile, then the V tile.
  auto step = [&](int t, int tn, lds_char* krd, lds_char* vrd, lds_char* kwr, lds_char* vwr) {
    if (tn < ntiles) {
      if constexpr (DIRECT) {
        dma_tile(tn, kwr, vwr);
      } else {
        load_stage(tn);
      }
    }
    if (t * C::BN < w_kend && (t + 1) * C::BN > w_kbeg) {
      Scores sc;
      tile_scores(krd, sc);
      if (tile_needs_mask(t)) tile_mask(t, sc);
      tile_softmax_pv(sc, vrd);
    }
    if constexpr (!DIRECT) {
      if (tn < ntiles) store_stage(kwr, vwr);
    }
    __syncthreads();
  };
  int t = next_tile(t_first);
  if (t < ntiles) {
    if constexpr (DIRECT) {
      dma_tile(t, k0s, v0s);
    } else {
      load_stage(t);
      store_stage(k0s, v0s);
    }
  }
  __syncthreads();
  while (t < ntiles) {
    int tn = next_tile(t + 1);
    step(t, tn, k0s, v0s, k1s, v1s);
    t = tn;
    if (t >= ntiles) break;
    tn = next_tile(t + 1);
    step(t, tn, k1s, v1s, k0s, v0s);
    t = tn;
  }

  // ---- epilogue: O = acc / l, or the partial of this key split -------------
  // In-kernel merge of the key splits (16-row waves only: the decode of
  // large groups): the partials of this position block go through
  // device-scope stores to a region of `prows` rows x S splits.
  const bool fused = (QBO == 1) && a.splits > 1 && a.counters != nullptr;
  const int prows = max(0, min(PB, N - p0));
  const uint32_t prow_bytes = (uint32_t)a.splits * (uint32_t)(D + 4) * 4u;
  const size_t orow0 = ((size_t)b * a.H + h) * N + p0;  // the block's first output row
  const __amdgpu_buffer_rsrc_t prs =
      raw_rsrc(fused ? (const void*)(a.partials + orow0 * a.splits * (size_t)(D + 4)) : a.out,
               fused ? (uint32_t)prows * prow_bytes : 0u);
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const float lt = H16 ? lacc[qb][0] : rows_sum(l_run[qb]);
    const int pos = wp0 + 16 * qb + c16;
    if (pos >= N) continue;
    if (a.splits > 1) {
      // record [m, l, -, -, acc[0..D)] of this row and split; m is the
      // softmax reference the weights were taken against
      if constexpr (QBO == 1) {
        if (fused) {
          const uint32_t ro = (uint32_t)(pos - p0) * prow_bytes + blockIdx.y * (uint32_t)(D + 4) * 4u;
          // words 2 and 3 of a record are zero: in row 0 they are the split's
          // go and claim words of the merge below, cleared here before the
          // ticket of this call
          if (qg == 0) st_dev4(prs, ro, f32x4{m_run[qb], lt, 0.f, 0.f});
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const int d = 16 * db + 4 * qg;
            if (d < D) st_dev4(prs, ro + 16u + 4u * d, acc[qb][db]);
          }
          continue;
        }
      }
      const size_t row = ((size_t)b * a.H + h) * N + pos;
      float* part = a.partials + (row * a.splits + blockIdx.y) * (size_t)(D + 4);
      if (qg == 0) {
        part[0] = m_run[qb];
        part[1] = lt;
      }
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const int d = 16 * db + 4 * qg;
        if (d < D) *reinterpret_cast<f32x4*>(part + 4 + d) = acc[qb][db];
      }
      continue;
    }
    const size_t obase = (((size_t)b * a.H + h) * N + pos) * (size_t)D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      const int d = 16 * db + 4 * qg;
      if (d >= D) continue;
      // a true division (not a reciprocal multiply) keeps l*x/l == x exact;
      // a row with no visible key has l == 0 and acc == 0, giving NaN
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = acc[qb][db][e] / lt;
      if constexpr (OUTF32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + obase + d) = o;
      } else {
        u32x2 pk = {pack16<ET>(o[0], o[1]), pack16<ET>(o[2], o[3])};
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + obase + d) = pk;
      }
    }
  }

  if constexpr (QBO == 1) {
    if (!fused) return;
    // ---- in-kernel merge of the key splits of this position block ---------
    // The S workgroups of the block (grid column y = split) share arrival
    // counter `arrive`; split s also owns two words of its row-0 partial
    // record, go (word 2) and claim (word 3), zeroed with its partial.  Each
    // workgroup stores its partial (device scope, complete before its
    // ticket), then takes a ticket.  The last to arrive knows every partial
    // is stored: it resets the counter, sets every other split's go word and
    // merges its own slice of rows.  The others poll their own go word (each
    // a different address), within a bounded spin: one that sees it sets its
    // claim to 1 and merges its slice; one that gives up sets it to 2 and
    // ends.  The last then waits for every claim (those splits hold tickets,
    // so they are running, and each claim comes within its bounded spin) and
    // merges the slices left to it.  Every output row is merged once (or,
    // only if a claim comes later than even the last's longer bound, twice
    // with identical values), whether or not the block's workgroups run at
    // the same time.
    const int S = a.splits;
    const int sp = (int)blockIdx.y;
    unsigned* const arrive = a.counters + L;      // merge group: (unit, position block)
    const size_t rec = (size_t)(D + 4);           // floats per partial record
    unsigned* const flags0 = reinterpret_cast<unsigned*>(a.partials + orow0 * S * rec) + 2;
    const int rs = (prows + S - 1) / S;           // rows per slice
    __shared__ int s_mode;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);         // this wave's partial stores are complete
    __syncthreads();
    if (tid == 0) {
      const unsigned t = __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
      int mode = 2;                               // 2: last, 1: merge own slice, 0: leave
      if (t == (unsigned)S - 1u) {
        st_dev(arrive, 0u);                       // ready for the next call
      } else {
        unsigned* const mine = flags0 + (size_t)sp * rec;
        unsigned go = __hip_atomic_load(mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int it = 0; go == 0u && it < kMergeSpin; ++it) {
          __builtin_amdgcn_s_sleep(2);
          go = __hip_atomic_load(mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        mode = go != 0u ? 1 : 0;
        st_dev(mine + 1, mode ? 1u : 2u);
      }
      s_mode = mode;
    }
    __syncthreads();
    const int mode = s_mode;
    if (mode == 0) return;
    if (mode == 2) {
      for (int i = tid; i < S; i += C::THREADS)
        if (i != sp) st_dev(flags0 + (size_t)i * rec, 1u);
    }
    merge_block_rows<ET, OUTF32>(a, prs, orow0, sp * rs, min(prows, (sp + 1) * rs), S, D, tid,
                                 C::THREADS);
    if (mode != 2) return;
    for (int i = tid; i < S; i += C::THREADS) {
      if (i == sp) continue;
      unsigned* const cl = flags0 + (size_t)i * rec + 1;
      unsigned c = __hip_atomic_load(cl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int it = 0; c == 0u && it < 4 * kMergeSpin; ++it) {
        __builtin_amdgcn_s_sleep(2);
        c = __hip_atomic_load(cl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (c != 1u)  // left to the last workgroup: this thread merges it alone
        merge_block_rows<ET, OUTF32>(a, prs, orow0, i * rs, min(prows, (i + 1) * rs), S, D, 0, 1);
    }
  }
}

// Merge the key-split partials of every query row, in split order, eight
// splits per memory round trip (indexes clamped to the last split): a
// running m*, with o = sum_s acc_s 2^((m_s - m*) sl) / sum_s l_s 2^((m_s - m*) sl).
constexpr int kMergeThreads = 128;
template <int ET, bool OUTF32>
__global__ void __launch_bounds__(kMergeThreads) prefill_merge_kernel(PrefillArgs a) {
  const size_t row = (size_t)blockIdx.x + (size_t)gridDim.x * blockIdx.z;
  const int d = blockIdx.y * kMergeThreads + threadIdx.x;
  if (d >= a.D || row >= (size_t)a.B * a.H * a.N) return;
  const float sl = kLog2e / sqrtf((float)a.D);
  const size_t stride = (size_t)a.D + 4;
  const int S = a.splits;
  const float* p = a.partials + row * S * stride;
  float mx = kNegInf, L = 0.f, A = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float pm[8], pl[8], pa[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t o = (size_t)min(s0 + u, S - 1) * stride;
      pm[u] = p[o];
      pl[u] = p[o + 1];
      pa[u] = p[o + 4 + d];
    }
    float cm = kNegInf;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < S) cm = fmaxf(cm, pm[u]);
    const float nm = fmaxf(mx, cm);
    if (nm == kNegInf) continue;                 // nothing visible yet
    const float f0 = (mx == kNegInf) ? 0.f : exp2_hw((mx - nm) * sl);
    L *= f0;
    A *= f0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (s0 + u < S) {
        const float f = exp2_hw((pm[u] - nm) * sl);
        L = fmaf(pl[u], f, L);
        A = fmaf(pa[u], f, A);
      }
    }
    mx = nm;
  }
  const float o = A / L;
  if constexpr (OUTF32) {
    reinterpret_cast<float*>(a.out)[row * a.D + d] = o;
  } else {
    reinterpret_cast<uint16_t*>(a.out)[row * a.D + d] = cvt16<ET>(o);
  }
}

// Workgroups of `threads` threads of `kernel` that the current device holds
// at once (occupancy per CU x CUs), looked up once per kernel and device
// (`cache`: one entry per device, owned by the caller's kernel instance, 0
// until looked up); 0 when the runtime cannot tell.
constexpr int kDevs = 64;
inline long resident_workgroups(const void* kernel, int threads, std::atomic<long>* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kDevs) {
    const long c = cache[dev].load(std::memory_order_relaxed);
    if (c != 0) return c;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  const long r = (long)per_cu * cus;
  if (dev >= 0 && dev < kDevs && r > 0) cache[dev].store(r, std::memory_order_relaxed);
  return r;
}

template <int ET, int DP, bool DIRECT, bool MASKED, bool OUTF32, int QBO>
hipError_t launch_k(const PrefillArgs& a, hipStream_t stream) {
  using C = PreCfg<ET != kF32, DP, QBO>;
  const int HG = (a.g % 4 == 0) ? 4 : ((a.g % 2 == 0) ? 2 : 1);
  const int PB = (C::NW / HG) * C::RW;
  const int npb = (a.N + PB - 1) / PB;
  const int units = a.B * a.H_kv * (a.g / HG);
  const long blocks = (long)npb * units;
  int order = (GQA_PREFILL_XCD_MAJOR && units % 8 == 0) ? 1 : 0;
  if (order && GQA_PREFILL_XCD_LPT && a.wr >= 0 && a.wl < 0) {
    // causal-type band: block weights grow with the block's last visible key
    const long long first = (long long)min(PB, a.N) - 1 + a.q_offset + a.wr + 1;
    const long long last = (long long)a.N - 1 + a.q_offset + a.wr + 1;
    if (2 * max(first, 1LL) <= min(last, (long long)a.M)) order = 2;
  }
  // The key splits merge inside the kernel (16-row waves only) when the
  // counter area holds an arrival counter per position block and every
  // workgroup of the launch can be resident at once (the
  // splits of a block wait for each other; the wait is bounded, but only
  // co-resident splits make it short).  Otherwise a second kernel merges.
  PrefillArgs ka = a;
  bool fused = false;
  if constexpr (QBO == 1) {
    static std::atomic<long> resident[kDevs];  // this kernel instance's occupancy per device
    fused = a.splits > 1 && a.counters != nullptr &&
            (long)units * npb <= (long)kMaxCounters &&
            blocks * a.splits <= resident_workgroups(
                                     (const void*)prefill_kernel<ET, DP, DIRECT, MASKED, OUTF32, QBO>,
                                     C::THREADS, resident);
  }
  if (!fused) ka.counters = nullptr;
  hipLaunchKernelGGL((prefill_kernel<ET, DP, DIRECT, MASKED, OUTF32, QBO>),
                     fold_grid(blocks, (unsigned)a.splits), dim3(C::THREADS), 0, stream, ka, HG,
                     units, npb, order);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1 || fused) return e;
  const long rows = (long)a.B * a.H * a.N;
  hipLaunchKernelGGL((prefill_merge_kernel<ET, OUTF32>),
                     fold_grid(rows, (unsigned)((a.D + kMergeThreads - 1) / kMergeThreads)),
                     dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

template <int ET, int DP, bool OUTF32, int QBO = 0>
hipError_t launch_dp(const PrefillArgs& a, hipStream_t stream) {
  if constexpr (ET != kF32) {
    if (a.D == DP) {
      return a.mask ? launch_k<ET, DP, true, true, OUTF32, QBO>(a, stream)
                    : launch_k<ET, DP, true, false, OUTF32, QBO>(a, stream);
    }
  }
  return a.mask ? launch_k<ET, DP, false, true, OUTF32, QBO>(a, stream)
                : launch_k<ET, DP, false, false, OUTF32, QBO>(a, stream);
}

template <int ET, bool OUTF32>
hipError_t launch_t(const PrefillArgs& a, hipStream_t stream) {
  if constexpr (ET == kF32) {
    if (a.D <= 16) return launch_dp<ET, 16, OUTF32>(a, stream);
  }
  if (a.D <= 32) return launch_dp<ET, 32, OUTF32>(a, stream);
  if (a.D <= 64) return launch_dp<ET, 64, OUTF32>(a, stream);
  if constexpr (ET != kF32) {
    // 16-row waves for the decode of large groups: a 64-head group fills one
    // block of four waves (with 32-row waves half of them would have no row)
    if (a.rows16 && a.D <= 128) return launch_dp<ET, 128, OUTF32, 1>(a, stream);
  }
  if (a.D <= 128) return launch_dp<ET, 128, OUTF32>(a, stream);
  return launch_dp<ET, 256, OUTF32>(a, stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
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
