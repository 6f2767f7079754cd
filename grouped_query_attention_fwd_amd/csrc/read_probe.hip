// HBM read-rate probe for gfx950 (measurement support, not part of the
// attention path).  Plain kernels that only stream a buffer with 16-byte
// loads, in the two access orders a decode can use, so the benchmark can
// state the read rate a simple kernel reaches on the GPU it runs on:
//   mode 0 (slabs): workgroup w reads its own contiguous slab of bytes / wgs,
//     front to back, like a decode workgroup reading its key range;
//   mode 1 (sweep): all workgroups sweep the buffer together, workgroup w
//     taking every wgs-th run of 256 * unroll * 16 bytes.
// Each thread XORs what it loads into one register and stores it only if it
// equals a value the data never produces, so no load can be dropped and
// nothing is written.  Built into its own library (libgqa_probe.so).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr uint32_t kNever = 0x9e3779b9u;   // the probe buffers hold ones

template <int UNROLL, bool NT>
__device__ __forceinline__ uint32_t fold(const u32x4* p, size_t i, size_t n) {
  uint32_t acc = 0;
  u32x4 v[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const size_t idx = i + (size_t)u * kThreads;
    const size_t c = idx < n ? idx : n - 1;   // clamped: loads stay in bounds
    v[u] = NT ? __builtin_nontemporal_load(p + c) : p[c];
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  return acc;
}

template <int UNROLL, bool NT>
__global__ void __launch_bounds__(kThreads) read_slabs(const u32x4* __restrict__ p, size_t n,
                                                       uint32_t* out) {
  const size_t per = (n + gridDim.x - 1) / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * per;
  const size_t hi = lo + per < n ? lo + per : n;
  uint32_t acc = 0;
  for (size_t i = lo + threadIdx.x; i < hi; i += (size_t)kThreads * UNROLL)
    acc ^= fold<UNROLL, NT>(p, i, hi);
  if (acc == kNever) out[blockIdx.x * kThreads + threadIdx.x] = acc;
}

template <int UNROLL, bool NT>
__global__ void __launch_bounds__(kThreads) read_sweep(const u32x4* __restrict__ p, size_t n,
                                                       uint32_t* out) {
  const size_t run = (size_t)kThreads * UNROLL;
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * run + threadIdx.x; i < n; i += (size_t)gridDim.x * run)
    acc ^= fold<UNROLL, NT>(p, i, n);
  if (acc == kNever) out[blockIdx.x * kThreads + threadIdx.x] = acc;
}

template <int UNROLL, bool NT>
hipError_t launch(int mode, const u32x4* p, size_t n, int wgs, uint32_t* out, hipStream_t s) {
  if (mode == 0) {
    hipLaunchKernelGGL((read_slabs<UNROLL, NT>), dim3(wgs), dim3(kThreads), 0, s, p, n, out);
  } else {
    hipLaunchKernelGGL((read_sweep<UNROLL, NT>), dim3(wgs), dim3(kThreads), 0, s, p, n, out);
  }
  return hipGetLastError();
}

}  // namespace

// Read `bytes` bytes at `buf` (device memory, 16-byte aligned, bytes a
// multiple of 16) once with `wgs` workgroups of 256 threads.  mode 0: one
// contiguous slab per workgroup; mode 1: all workgroups sweep together.
// unroll: 4, 8 or 16 loads in flight per thread.  nt: non-temporal loads.
// out: device buffer of wgs * 256 uint32 that is never written in practice.
// Returns 0 on success, 1 for bad arguments, 2 for a launch error.
extern "C" int gqa_probe_read(const void* buf, size_t bytes, int wgs, int mode, int unroll, int nt,
                              void* out, void* stream) {
  if (buf == nullptr || out == nullptr || bytes < 16 || bytes % 16 != 0 || wgs < 1 ||
      wgs > 65536 || (mode != 0 && mode != 1) || ((uintptr_t)buf & 15u) != 0)
    return 1;
  const u32x4* p = static_cast<const u32x4*>(buf);
  const size_t n = bytes / 16;
  uint32_t* o = static_cast<uint32_t*>(out);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  switch (unroll * 2 + (nt ? 1 : 0)) {
    case 8: e = launch<4, false>(mode, p, n, wgs, o, s); break;
    case 9: e = launch<4, true>(mode, p, n, wgs, o, s); break;
    case 16: e = launch<8, false>(mode, p, n, wgs, o, s); break;
    case 17: e = launch<8, true>(mode, p, n, wgs, o, s); break;
    case 32: e = launch<16, false>(mode, p, n, wgs, o, s); break;
    case 33: e = launch<16, true>(mode, p, n, wgs, o, s); break;
    default: return 1;
  }
  return e == hipSuccess ? 0 : 2;
}
