// Device-side helpers shared by the decode and prefill kernels (gfx950).
//
// MFMA lane layouts used throughout (wave64, checked on the hardware):
//   v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8*(l/16)+s] and
//     B[8*(l/16)+s][l%16] for s = 0..7; the result lane l, register r holds
//     C[4*(l/16)+r][l%16].
//   v_mfma_f32_16x16x4f32: lane l holds A[l%16][l/16] and B[l/16][l%16];
//     the result uses the same C layout.
//   v_mfma_f32_16x16x32_f16: the same layout as the bf16 form.
// Both attention products are formed transposed, S^T = K Q^T and
// O^T = V^T P^T, so a lane always owns one query (or one query head) in the
// column index l%16 and four consecutive keys (or d) in its registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) char lds_char;

// Element types of q, k and v (values of the C ABI's gqa_dtype_t).
enum : int { kF32 = 0, kBF16 = 1, kF16 = 2 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Hardware 2^x (v_exp_f32).  exp2(-inf) = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Device-scope (all XCDs) relaxed store: coherent across the per-XCD L2s
// without a cache write-back or invalidation.
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Raw buffer descriptor over `bytes` bytes at `base` (gfx9 descriptor
// format word).  Accesses past `bytes` are dropped: loads return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// Cache-policy operand of a device-scope access (the sc1 bit): like st_dev,
// coherent across the XCDs' L2s.
constexpr int kCpolDevice = 16;
__device__ __forceinline__ f32x4 ld_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolDevice));
}
__device__ __forceinline__ f32x2 ld_dev2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCpolDevice));
}
__device__ __forceinline__ void st_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, kCpolDevice);
}
__device__ __forceinline__ void st_dev2(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x2 x) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), r, off, 0, kCpolDevice);
}
// s_waitcnt immediate (gfx9 layout) that waits for every vector memory
// access of the wave, loads and stores, to complete: vmcnt 0, expcnt and
// lgkmcnt at their maximum (no wait).
constexpr int kWaitVm0 = (0x7 << 4) | (0xF << 8);

// bf16 (stored as raw 16-bit) to fp32: the bf16 bits are the high half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16x2 (v_cvt_pk_bf16_f32: round to nearest, ties to
// even; NaN stays NaN).  `lo` lands in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return (uint16_t)(pack_bf16x2(f, 0.f) & 0xffffu);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---- 16-bit element types (ET = kBF16 or kF16) -------------------------
// 16x16x32 matrix-core product on operands held as raw 16-byte words.
template <int ET>
__device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
  static_assert(ET == kBF16 || ET == kF16, "16-bit element types only");
  if constexpr (ET == kBF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Two fp32 -> one packed pair of ET (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32:
// round to nearest, ties to even).  `lo` lands in the low half.
template <int ET>
__device__ __forceinline__ uint32_t pack16(float lo, float hi) {
  if constexpr (ET == kBF16) return pack_bf16x2(lo, hi);
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

template <int ET>
__device__ __forceinline__ uint16_t cvt16(float f) {
  return (uint16_t)(pack16<ET>(f, 0.f) & 0xffffu);
}

// Eight fp32 values -> one 16-byte MFMA operand of ET.
template <int ET>
__device__ __forceinline__ u32x4 pack16x8(const float* x) {
  u32x4 w;
  w[0] = pack16<ET>(x[0], x[1]);
  w[1] = pack16<ET>(x[2], x[3]);
  w[2] = pack16<ET>(x[4], x[5]);
  w[3] = pack16<ET>(x[6], x[7]);
  return w;
}

// 16-byte global load (caller guarantees 16-byte alignment).
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// 16-byte global load with the non-temporal hint (global_load_dwordx4 ...
// nt): for data read once per call, such as a decode's K/V stream.  Measured
// on MI355X: plain streaming reads of 268 MB and 2 GiB reach 6.9 and 7.2 TB/s
// with the hint against 6.2 and 6.4 TB/s without it.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ u32x4 sel16(bool keep, u32x4 v) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = keep ? v[i] : 0u;
  return r;
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4).
// The LDS destination is `lds_base` + 16 * lane: `lds_base` must be the same
// for the whole wave; each lane chooses its global source freely.
__device__ __forceinline__ void dma16(const void* gsrc, lds_char* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// LDS accessors on a byte offset into a shared buffer.
__device__ __forceinline__ void lds_st16(lds_char* base, uint32_t off, u32x4 v) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(base + off) = v;
}
__device__ __forceinline__ u32x4 lds_ld16(const lds_char* base, uint32_t off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(base + off);
}
__device__ __forceinline__ float lds_ldf(const lds_char* base, uint32_t off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) float*>(base + off);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// the 16 eight-byte addresses are taken as a 4 x 16 block of 16-bit values
// (lanes 4r..4r+3 address row r, columns 4*(lane%4)..+3); lane c of the
// group receives column c, rows 0..3.
__device__ __forceinline__ i16x4 lds_ld_tr16(lds_char* base, uint32_t off) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off));
}

// Two transposed reads -> one 16-byte operand (any 16-bit element type).
__device__ __forceinline__ u32x4 concat16(i16x4 a, i16x4 b) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(u32x4, c);
}

// Cross-lane reductions inside a wave.
__device__ __forceinline__ float shfl_xor_f(float x, int m) { return __shfl_xor(x, m, 64); }

// Reduce over the four 16-lane rows of a wave (lanes c, c+16, c+32, c+48),
// every lane receiving the result.  v_permlane16_swap / v_permlane32_swap
// exchange rows between two registers; called with the same value twice,
// the two results hold the two halves of each pair, so combining them gives
// the pairwise reduction whichever half lands where.  VALU only, no LDS.
__device__ __forceinline__ float rows_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// Sum of an int over the 64 lanes of a wave, in every lane: DPP adds inside
// each 16-lane row (quad swaps, then the half-row and row mirrors), then the
// two row swaps.  Every lane must be active.
__device__ __forceinline__ int wave_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  x += __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  x += __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false);  // row_mirror
  auto a = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
  x = (int)(a[0] + a[1]);
  auto b = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return (int)(b[0] + b[1]);
}
// Maximum of an int over the 64 lanes of a wave, in every lane (the same
// steps as wave_sum).
__device__ __forceinline__ int wave_max(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false));
  auto a = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
  x = max((int)a[0], (int)a[1]);
  auto b = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return max((int)b[0], (int)b[1]);
}
// Inclusive prefix sum of an int over the 64 lanes of a wave: DPP row
// shifts by 1, 2, 4 and 8 inside each 16-lane row (lanes shifted in from
// outside the row add zero), then lane 15 of each row is added to the next
// row and lane 31 to the upper half.  Every lane must be active.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
  return x;
}
__device__ __forceinline__ float rows_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace gqa
