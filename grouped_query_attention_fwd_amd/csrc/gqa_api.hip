// C ABI of libgqa.so: argument validation, workspace sizing and dispatch.
// Every check runs on the host before any HIP call, so a rejected call has
// no side effect.  The declarations and their contract live in include/gqa.h.
#include "../../include/gqa.h"
#include "gqa_internal.h"

static_assert(gqa::kCounterBytes == GQA_DECODE_COUNTER_BYTES, "counter area size");
static_assert(sizeof(gqa_status_t) == sizeof(int) && sizeof(gqa_dtype_t) == sizeof(int),
              "the C ABI's enums are int-sized");

#include <limits.h>

#include <initializer_list>
#include <mutex>

// The fixed scratch area of gqa_decode_noalloc: arrival counters, then the
// key-split partials, as in a gqa_decode workspace.
constexpr size_t kScratchBytes = GQA_DECODE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t dtype_size(gqa_dtype_t t) { return t == GQA_F32 ? 4 : 2; }

bool dtype_ok(gqa_dtype_t t) { return t == GQA_F32 || t == GQA_BF16 || t == GQA_F16; }

// [lo, lo + n) overlaps [p, p + m)?
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Product of non-negative factors, or -1 on int64 overflow.
long long mul_checked(std::initializer_list<long long> xs) {
  long long r = 1;
  for (long long x : xs) {
    if (x < 0) return -1;
    if (x != 0 && r > LLONG_MAX / x) return -1;
    r *= x;
  }
  return r;
}

gqa_status_t check_common(const void* q, const void* k, const void* v, const void* out, int B,
                          int H, int H_kv, int N, int M, int D, gqa_dtype_t in_dtype,
                          gqa_dtype_t out_dtype) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return GQA_ERR_NULL;
  if (B < 1 || H < 1 || H_kv < 1 || N < 1 || M < 1 || D < 1) return GQA_ERR_SHAPE;
  if (H % H_kv != 0) return GQA_ERR_GROUP;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return GQA_ERR_DTYPE;
  if (out_dtype != in_dtype && out_dtype != GQA_F32) return GQA_ERR_DTYPE;
  if (D > 256 || (D * dtype_size(in_dtype)) % 16 != 0) return GQA_ERR_UNSUPPORTED;
  // row counts must stay below 2^31 and element counts within int64
  const long long qrows = mul_checked({B, H, N});
  const long long kvrows = mul_checked({B, H_kv, M});
  const long long mask_elems = mul_checked({B, N, M});
  if (qrows < 0 || kvrows < 0 || mask_elems < 0 || qrows >= INT_MAX || kvrows >= INT_MAX)
    return GQA_ERR_SHAPE;
  if (mul_checked({qrows, D, 4}) < 0 || mul_checked({kvrows, D, 4}) < 0) return GQA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return GQA_ERR_ALIGN;
  return GQA_OK;
}


// out must not overlap q, k, v or the mask of a decode call.
gqa_status_t check_decode_alias(const void* q, const void* k, const void* v, const uint8_t* mask,
                                const void* out, int B, int H, int H_kv, int M, int D,
                                gqa_dtype_t in_dtype, gqa_dtype_t out_dtype) {
  const size_t ein = dtype_size(in_dtype), eout = dtype_size(out_dtype);
  const size_t qb = (size_t)B * H * D * ein, kvb = (size_t)B * H_kv * M * D * ein;
  const size_t ob = (size_t)B * H * D * eout;
  if (overlaps(out, ob, q, qb) || overlaps(out, ob, k, kvb) || overlaps(out, ob, v, kvb) ||
      overlaps(out, ob, mask, (size_t)B * M))
    return GQA_ERR_ALIAS;
  return GQA_OK;
}

#if GQA_DECODE_TRACE
// Timing build: where decode workgroups write their records (null: off).
void* g_decode_trace = nullptr;
#endif

// Launch a validated decode with its plan; `workspace` holds at least
// plan.workspace_bytes bytes (counter area first) when that is nonzero.
gqa_status_t launch_decode_plan(const gqa::DecodePlan& plan, const void* q, const void* k,
                                const void* v, const uint8_t* mask, void* out, int B, int H,
                                int H_kv, int M, int D, gqa_dtype_t in_dtype,
                                gqa_dtype_t out_dtype, void* workspace, void* stream) {
  if (plan.wide) {
    // the group's heads as the query rows of a prefill over the same K/V:
    // q [B, H, 1, D] is [B, H_kv, g, D]; the [B, 1, M] mask serves every row
    gqa::PrefillArgs p{};
    p.q = q; p.k = k; p.v = v; p.mask = mask; p.out = out;
    p.B = B; p.H = H_kv; p.H_kv = H_kv; p.N = H / H_kv; p.M = M; p.D = D;
    p.g = 1;
    p.q_offset = 0; p.wl = -1; p.wr = -1;
    p.mask_rs = 0;
    p.mask_bs = M;
    p.splits = plan.wide_splits;
    p.kps = plan.wide_kps;
    p.rows16 = 1;
    p.partials = plan.workspace_bytes > 0
                     ? reinterpret_cast<float*>(static_cast<char*>(workspace) + gqa::kCounterBytes)
                     : nullptr;
    p.counters = plan.workspace_bytes > 0 ? reinterpret_cast<unsigned*>(workspace) : nullptr;
    p.in_type = (int)in_dtype;
    p.out_f32 = out_dtype == GQA_F32;
    if (gqa::launch_prefill(p, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return GQA_ERR_HIP;
    return GQA_OK;
  }

  gqa::DecodeArgs a{};
  a.q = q; a.k = k; a.v = v; a.mask = mask; a.out = out;
  a.B = B; a.H = H; a.H_kv = H_kv; a.M = M; a.D = D;
  a.g = H / H_kv;
  a.head_chunk = plan.head_chunk;
  a.head_chunks = plan.head_chunks;
  a.xcd_group = plan.xcd_group;
  a.splits = plan.splits;
  a.keys_per_split = plan.keys_per_split;
  // a rotated key walk measured 4-7 % faster for caches of 8 MB or more per
  // KV head (all split ranges then start at equally aligned addresses) and
  // about 1 % slower for smaller ones
  a.rotate = (size_t)M * D * dtype_size(in_dtype) >= ((size_t)8 << 20) ? 1 : 0;
  a.in_type = (int)in_dtype;  // gqa_dtype_t values match kF32 / kBF16 / kF16
  a.out_f32 = out_dtype == GQA_F32;
  if (plan.workspace_bytes > 0) {
    a.counters = reinterpret_cast<unsigned*>(workspace);
    a.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + gqa::kCounterBytes);
  }
#if GQA_DECODE_TRACE
  a.trace = static_cast<unsigned long long*>(g_decode_trace);
#endif
  if (gqa::launch_decode(a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return GQA_ERR_HIP;
  return GQA_OK;
}

// ---- the fixed scratch area of gqa_decode_noalloc ----------------------------
// Each GPU holds its own copy of this array from the moment the library's
// code is loaded on it until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol): it uses the device address that hipGetSymbolAddress returns, kept
// per device.
static_assert(kScratchBytes > gqa::kCounterBytes, "scratch holds the counter area");

__global__ void clear_words(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's scratch array, or null when the
// HIP runtime reports an error.  The first call on a device looks the address
// up and clears the arrival counters with a small kernel on `stream`.
void* scratch_for_current_device(hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&]() {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return;
    const int words = (int)(gqa::kCounterBytes / 4);
    hipLaunchKernelGGL(clear_words, dim3((words + 255) / 256), dim3(256), 0, stream,
                       static_cast<unsigned*>(p), words);
    if (hipGetLastError() != hipSuccess) return;
    slot.ptr = p;
  });
  return slot.ptr;
}

}  // namespace

extern "C" {

const char* gqa_status_string(gqa_status_t s) {
  switch (s) {
    case GQA_OK: return "success";
    case GQA_ERR_NULL: return "a required pointer is NULL";
    case GQA_ERR_SHAPE: return "invalid shape (a dimension < 1, or sizes exceed the limits)";
    case GQA_ERR_GROUP: return "H is not a multiple of H_kv";
    case GQA_ERR_DTYPE: return "unsupported dtype combination";
    case GQA_ERR_ALIGN: return "q/k/v/out/workspace must be 16-byte aligned";
    case GQA_ERR_UNSUPPORTED:
      return "unsupported size (need D <= 256, D*sizeof(dtype) % 16 == 0 and, paged, block_size % 16 == 0)";
    case GQA_ERR_WORKSPACE: return "decode workspace missing or too small";
    case GQA_ERR_HIP: return "HIP runtime error";
    case GQA_ERR_ALIAS: return "out overlaps an input or the workspace";
    case GQA_ERR_SCRATCH:
      return "the problem needs more scratch than gqa_decode_noalloc holds "
             "(GQA_DECODE_NOALLOC_SCRATCH_BYTES); use gqa_decode with a workspace";
  }
  return "unknown status";
}

size_t gqa_decode_workspace_size(int B, int H, int H_kv, int M, int D) {
  if (B < 1 || H < 1 || H_kv < 1 || M < 1 || D < 1 || H % H_kv != 0) return 0;
  const long long kvrows = mul_checked({B, H_kv, M});
  if (kvrows < 0 || kvrows >= INT_MAX || mul_checked({B, H}) >= INT_MAX) return 0;
  return gqa::plan_decode(B, H, H_kv, M, D, false).workspace_bytes;
}

gqa_status_t gqa_decode(const void* q, const void* k, const void* v, const uint8_t* mask,
                        void* out, int B, int H, int H_kv, int M, int D, gqa_dtype_t in_dtype,
                        gqa_dtype_t out_dtype, void* workspace, size_t workspace_bytes,
                        void* stream) {
  gqa_status_t st = check_common(q, k, v, out, B, H, H_kv, 1, M, D, in_dtype, out_dtype);
  if (st != GQA_OK) return st;
  const gqa::DecodePlan plan = gqa::plan_decode(B, H, H_kv, M, D, false);
  if (plan.workspace_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < plan.workspace_bytes) return GQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return GQA_ERR_ALIGN;
  }
  st = check_decode_alias(q, k, v, mask, out, B, H, H_kv, M, D, in_dtype, out_dtype);
  if (st != GQA_OK) return st;
  if (plan.workspace_bytes > 0 && overlaps(out, (size_t)B * H * D * dtype_size(out_dtype),
                                           workspace, plan.workspace_bytes))
    return GQA_ERR_ALIAS;
  return launch_decode_plan(plan, q, k, v, mask, out, B, H, H_kv, M, D, in_dtype, out_dtype,
                            workspace, stream);
}

gqa_status_t gqa_decode_noalloc(const void* q, const void* k, const void* v, const uint8_t* mask,
                                void* out, int B, int H, int H_kv, int M, int D,
                                gqa_dtype_t in_dtype, gqa_dtype_t out_dtype, void* stream) {
  gqa_status_t st = check_common(q, k, v, out, B, H, H_kv, 1, M, D, in_dtype, out_dtype);
  if (st != GQA_OK) return st;
  const gqa::DecodePlan plan = gqa::plan_decode(B, H, H_kv, M, D, false);
  if (plan.workspace_bytes > kScratchBytes) return GQA_ERR_SCRATCH;
  st = check_decode_alias(q, k, v, mask, out, B, H, H_kv, M, D, in_dtype, out_dtype);
  if (st != GQA_OK) return st;
  void* ws = nullptr;
  if (plan.workspace_bytes > 0) {
    // the first call on this device finds the device's copy of the array
    // and clears its counter area (on this stream, ahead of the decode)
    ws = scratch_for_current_device(reinterpret_cast<hipStream_t>(stream));
    if (ws == nullptr) return GQA_ERR_HIP;
  }
  return launch_decode_plan(plan, q, k, v, mask, out, B, H, H_kv, M, D, in_dtype, out_dtype, ws,
                            stream);
}

size_t gqa_decode_paged_workspace_size(int B, int H, int H_kv, int max_blocks, int block_size,
                                       int D) {
  const long long m = mul_checked({max_blocks, block_size});
  if (m < 1 || m >= INT_MAX) return 0;
  if (B < 1 || H < 1 || H_kv < 1 || D < 1 || H % H_kv != 0) return 0;
  const long long kvrows = mul_checked({B, H_kv, m});
  if (kvrows < 0 || kvrows >= INT_MAX || mul_checked({B, H}) >= INT_MAX) return 0;
  return gqa::plan_decode(B, H, H_kv, (int)m, D, true).workspace_bytes;
}

gqa_status_t gqa_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_table, const int32_t* kv_len, void* out,
                              int B, int H, int H_kv, int max_blocks, int block_size,
                              int num_blocks, int D, gqa_dtype_t in_dtype,
                              gqa_dtype_t out_dtype, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (block_table == nullptr || kv_len == nullptr) return GQA_ERR_NULL;
  if (max_blocks < 1 || block_size < 1 || num_blocks < 1) return GQA_ERR_SHAPE;
  if (block_size % 16 != 0) return GQA_ERR_UNSUPPORTED;
  const long long m = mul_checked({max_blocks, block_size});
  if (m < 1 || m >= INT_MAX) return GQA_ERR_SHAPE;
  const int M = (int)m;
  // the per-sequence view is [B, H_kv, M, D]; the pool has its own row count
  gqa_status_t st = check_common(q, k_pool, v_pool, out, B, H, H_kv, 1, M, D, in_dtype, out_dtype);
  if (st != GQA_OK) return st;
  const long long pool_rows = mul_checked({num_blocks, H_kv, block_size});
  if (pool_rows < 0 || mul_checked({pool_rows, D, 4}) < 0) return GQA_ERR_SHAPE;
  if (mul_checked({B, max_blocks}) >= INT_MAX) return GQA_ERR_SHAPE;
  if (((uintptr_t)block_table & 3u) != 0 || ((uintptr_t)kv_len & 3u) != 0) return GQA_ERR_ALIGN;
  const gqa::DecodePlan plan = gqa::plan_decode(B, H, H_kv, M, D, true);
  if (plan.workspace_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < plan.workspace_bytes) return GQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return GQA_ERR_ALIGN;
  }
  const size_t ein = dtype_size(in_dtype), eout = dtype_size(out_dtype);
  const size_t qb = (size_t)B * H * D * ein, poolb = (size_t)pool_rows * D * ein;
  const size_t ob = (size_t)B * H * D * eout;
  if (overlaps(out, ob, q, qb) || overlaps(out, ob, k_pool, poolb) ||
      overlaps(out, ob, v_pool, poolb) ||
      overlaps(out, ob, block_table, (size_t)B * max_blocks * 4) ||
      overlaps(out, ob, kv_len, (size_t)B * 4) ||
      (plan.workspace_bytes > 0 && overlaps(out, ob, workspace, plan.workspace_bytes)))
    return GQA_ERR_ALIAS;

  gqa::DecodeArgs a{};
  a.q = q; a.k = k_pool; a.v = v_pool; a.mask = nullptr; a.out = out;
  a.block_table = block_table; a.kv_len = kv_len;
  a.num_blocks = num_blocks; a.block_size = block_size; a.max_blocks = max_blocks;
  a.B = B; a.H = H; a.H_kv = H_kv; a.M = M; a.D = D;
  a.g = H / H_kv;
  a.head_chunk = plan.head_chunk;
  a.head_chunks = plan.head_chunks;
  a.xcd_group = plan.xcd_group;
  a.splits = plan.splits;
  a.keys_per_split = plan.keys_per_split;
  a.pieces = plan.pieces;
  a.in_type = (int)in_dtype;  // gqa_dtype_t values match kF32 / kBF16 / kF16
  a.out_f32 = out_dtype == GQA_F32;
  if (plan.workspace_bytes > 0) {
    a.counters = reinterpret_cast<unsigned*>(workspace);
    a.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + gqa::kCounterBytes);
  }
#if GQA_DECODE_TRACE
  a.trace = static_cast<unsigned long long*>(g_decode_trace);
#endif
  if (gqa::launch_decode(a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return GQA_ERR_HIP;
  return GQA_OK;
}

gqa_status_t gqa_prefill_band(const void* q, const void* k, const void* v, const uint8_t* mask,
                              void* out, int B, int H, int H_kv, int N, int M, int D,
                              int q_offset, int window_left, int window_right,
                              gqa_dtype_t in_dtype, gqa_dtype_t out_dtype, void* stream) {
  gqa_status_t st = check_common(q, k, v, out, B, H, H_kv, N, M, D, in_dtype, out_dtype);
  if (st != GQA_OK) return st;
  const size_t ein = dtype_size(in_dtype), eout = dtype_size(out_dtype);
  const size_t qb = (size_t)B * H * N * D * ein, kvb = (size_t)B * H_kv * M * D * ein;
  const size_t ob = (size_t)B * H * N * D * eout;
  if (overlaps(out, ob, q, qb) || overlaps(out, ob, k, kvb) || overlaps(out, ob, v, kvb) ||
      overlaps(out, ob, mask, (size_t)B * N * M))
    return GQA_ERR_ALIAS;

  gqa::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.mask = mask; a.out = out;
  a.B = B; a.H = H; a.H_kv = H_kv; a.N = N; a.M = M; a.D = D;
  a.g = H / H_kv;
  a.q_offset = q_offset;
  a.wl = window_left < 0 ? -1 : window_left;
  a.wr = window_right < 0 ? -1 : window_right;
  a.mask_rs = M;
  a.mask_bs = (long long)N * M;
  a.splits = 1;
  a.kps = M;
  a.in_type = (int)in_dtype;  // gqa_dtype_t values match kF32 / kBF16 / kF16
  a.out_f32 = out_dtype == GQA_F32;
  if (gqa::launch_prefill(a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return GQA_ERR_HIP;
  return GQA_OK;
}

gqa_status_t gqa_prefill(const void* q, const void* k, const void* v, const uint8_t* mask,
                         int causal, void* out, int B, int H, int H_kv, int N, int M, int D,
                         gqa_dtype_t in_dtype, gqa_dtype_t out_dtype, void* stream) {
  // causal: the band with no left limit and right edge at the query position
  return gqa_prefill_band(q, k, v, mask, out, B, H, H_kv, N, M, D, 0, -1, causal ? 0 : -1,
                          in_dtype, out_dtype, stream);
}

#if GQA_DECODE_TRACE
// Timing build only: set the buffer of kTraceRecords * 8 uint64 that the
// decode kernels fill (null turns the trace off), and report the frequency
// of the wall clock the records count, in kHz (0 on error).
void gqa_debug_decode_trace(void* buffer) { g_decode_trace = buffer; }
int gqa_debug_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}
#endif

}  // extern "C"
