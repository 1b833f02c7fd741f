// Split-KV paged decode for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation): the
// two-launch decode of mi_split_kv_decode with its fp32 partials kept in a
// static device array of the library instead of caller workspaces.
//
// The array lives in this file. Its name is only a host-side stand-in for
// the device symbol, so host code never passes it to a kernel: the device
// address is fetched once per device with hipGetSymbolAddress (with that
// device current) and that pointer is what the launches receive. Every GPU
// holds its own copy of the array until the process ends; all calls on one
// GPU share it, so calls that overlap on one GPU race on the partials.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "launch.h"
#include "mi.h"

namespace {
constexpr int kD = 128;
constexpr int64_t kScratchRows = MI_NOALLOC_MAX_PARTIAL_ROWS;
constexpr int kMaxDevices = 64;
}  // namespace

// Partial outputs [rows, D] followed by partial LSEs [rows], fp32.
static __device__ __align__(256) float scratch[kScratchRows * (kD + 1)];

namespace {

std::atomic<float*> g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`, looked up on the first call on
// that device (concurrent first calls store the same address).
mi_status scratch_for_current_device(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MI_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MI_ERR_UNSUPPORTED;
  float* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
      return MI_ERR_HIP;
    p = static_cast<float*>(addr);
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MI_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlaps(const void* p, int64_t n, const void* q, int64_t m) {
  if (p == nullptr || q == nullptr || n <= 0 || m <= 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uintptr_t b = reinterpret_cast<uintptr_t>(q);
  return a < b + static_cast<uintptr_t>(m) && b < a + static_cast<uintptr_t>(n);
}

}  // namespace

extern "C" mi_status mi_split_kv_decode_noalloc(
    const void* q, const void* k_cache, const void* v_cache, const int32_t* page_table,
    int32_t pt_stride, const int32_t* ctx_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
    int32_t page_size, int64_t num_phys_pages, int32_t num_splits, float sm_scale,
    mi_dtype kv_dtype, void* o, float* lse, mi_dtype out_dtype, void* stream) {
  if (!q || !k_cache || !v_cache || !page_table || !ctx_lens || !o) return MI_ERR_NULL;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || page_size <= 0 || pt_stride <= 0 ||
      num_phys_pages <= 0 || num_splits <= 0 || Hq % Hkv != 0)
    return MI_ERR_SHAPE;
  if (kv_dtype != MI_F16 && kv_dtype != MI_BF16) return MI_ERR_DTYPE;
  if (out_dtype != MI_F16 && out_dtype != MI_BF16 && out_dtype != MI_F32) return MI_ERR_DTYPE;
  const int G = Hq / Hkv;
  if (D != kD || page_size != 16 || !(G == 1 || G == 2 || G == 4 || G == 8) ||
      num_splits > 1024 || B > 65535 || Hkv > 65535)
    return MI_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(page_table, 4) || !aligned(ctx_lens, 4))
    return MI_ERR_UNSUPPORTED;
  const int64_t rows = int64_t(B) * Hq * num_splits;
  if (rows > kScratchRows) return MI_ERR_SCRATCH;
  if (num_phys_pages > (int64_t(1) << 62) / (int64_t(Hkv) * page_size * D * 2) ||
      int64_t(B) * pt_stride > (int64_t(1) << 60))
    return MI_ERR_SHAPE;
  const int64_t o_bytes = int64_t(B) * Hq * D * (out_dtype == MI_F32 ? 4 : 2);
  const int64_t lse_bytes = int64_t(B) * Hq * 4;
  const int64_t cache_bytes = num_phys_pages * Hkv * page_size * D * 2;
  const void* ins[5] = {q, k_cache, v_cache, page_table, ctx_lens};
  const int64_t in_b[5] = {int64_t(B) * Hq * D * 2, cache_bytes, cache_bytes,
                           int64_t(B) * pt_stride * 4, int64_t(B) * 4};
  for (int i = 0; i < 5; ++i)
    if (overlaps(o, o_bytes, ins[i], in_b[i]) || overlaps(lse, lse_bytes, ins[i], in_b[i]))
      return MI_ERR_ALIAS;
  if (overlaps(o, o_bytes, lse, lse_bytes)) return MI_ERR_ALIAS;
  if (B == 0) return MI_OK;
  float* base = nullptr;
  mi_status st = scratch_for_current_device(&base);
  if (st != MI_OK) return st;
  float* o_part = base;
  float* lse_part = base + kScratchRows * kD;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (num_splits == 1)  // one split: pass 1 writes o and lse itself
    return mi::launch_split_kv_partial(q, k_cache, v_cache, page_table, pt_stride, ctx_lens, B, Hq,
                                       Hkv, num_phys_pages, 1, sm_scale, kv_dtype, o_part,
                                       lse_part, hs, nullptr, o, lse, out_dtype) == hipSuccess
               ? MI_OK
               : MI_ERR_HIP;
  if (mi::launch_split_kv_partial(q, k_cache, v_cache, page_table, pt_stride, ctx_lens, B, Hq,
                                  Hkv, num_phys_pages, num_splits, sm_scale, kv_dtype, o_part,
                                  lse_part, hs) != hipSuccess)
    return MI_ERR_HIP;
  return mi::launch_merge_states(o_part, lse_part, o, lse, int64_t(B) * Hq, num_splits, 1, D,
                                 MI_F32, out_dtype, hs) == hipSuccess
             ? MI_OK
             : MI_ERR_HIP;
}
