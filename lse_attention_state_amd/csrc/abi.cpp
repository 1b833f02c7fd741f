// C ABI of libmi.so: argument validation on the host, then kernel launches on
// the caller's stream. Nothing is allocated, freed or synchronised here.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "launch.h"
#include "mi.h"
#include "split_range.h"

namespace {

// Per-sequence split decode: sequences (the device-side segment search reads
// at most 64 entries per round, two rounds) and work items (grid height).
constexpr int32_t kMaxVarlenSeqs = 4031;
constexpr int32_t kMaxVarlenSplits = 65535;

bool dtype_ok(int dt) { return dt == MI_F16 || dt == MI_BF16 || dt == MI_F32; }

int64_t dtype_bytes(int dt) { return dt == MI_F32 ? 4 : 2; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte ranges [p, p + n) and [q, q + m) share a byte.
bool overlaps(const void* p, int64_t n, const void* q, int64_t m) {
  if (p == nullptr || q == nullptr || n <= 0 || m <= 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uintptr_t b = reinterpret_cast<uintptr_t>(q);
  return a < b + static_cast<uintptr_t>(m) && b < a + static_cast<uintptr_t>(n);
}

// An output may coincide exactly with one input (in-place) when `exact_ok`;
// any other shared byte is an aliasing error.
bool bad_alias(const void* out, int64_t out_bytes, const void* in, int64_t in_bytes, bool exact_ok) {
  if (!overlaps(out, out_bytes, in, in_bytes)) return false;
  return !(exact_ok && out == in && out_bytes == in_bytes);
}

// hipErrorInvalidConfiguration comes from a launcher's own check that the grid
// fits (nothing was launched): a size the library does not support.
mi_status from_hip(hipError_t e) {
  if (e == hipSuccess) return MI_OK;
  return e == hipErrorInvalidConfiguration ? MI_ERR_UNSUPPORTED : MI_ERR_HIP;
}

// Compute units of the current device, cached per device (the only state the
// library keeps; concurrent first calls store the same value).
mi_status device_cus(int* cus) {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MI_ERR_HIP;
  if (dev >= 0 && dev < 64 && cached[dev] > 0) {
    *cus = cached[dev];
    return MI_OK;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return MI_ERR_HIP;
  if (dev >= 0 && dev < 64) cached[dev] = n;
  *cus = n;
  return MI_OK;
}

// The single-launch decode pays, in every workgroup, a wait for its partials
// to complete and a device-scope counter update, and in the last workgroup of
// each (sequence, kv head) an L2 invalidation that the other workgroups' K/V
// streams feel. Measured on MI355X (the L3 page's three workloads and the
// mixed batch at 1-64 splits), it beats pass 1 plus a separate combine launch
// while the work items are at most twice the compute units, and loses beyond.
bool single_launch_pays(int64_t work_items, int cus) { return work_items <= 2 * int64_t(cus); }

// Products of validated non-negative sizes stay below 2^62 bytes.
bool size_ok(int64_t a, int64_t b, int64_t c = 1, int64_t d = 1) {
  const int64_t lim = int64_t(1) << 62;
  int64_t x = a;
  for (int64_t f : {b, c, d}) {
    if (f != 0 && x > lim / f) return false;
    x *= f;
  }
  return true;
}

mi_status check_merge_dims(int32_t H, int32_t D, int dt_in, int dt_out) {
  if (H <= 0 || D <= 0) return MI_ERR_SHAPE;
  if (!dtype_ok(dt_in) || !dtype_ok(dt_out)) return MI_ERR_DTYPE;
  if (D % 8 != 0 || D > 512) return MI_ERR_UNSUPPORTED;
  return MI_OK;
}

struct DecodeShape {
  int64_t q_bytes, cache_bytes, pt_bytes, ctx_bytes, opart_bytes, lpart_bytes;
};

// part_rows: partial states per query head (B * num_splits for the uniform
// layout; 0 means that, otherwise the per-sequence layout's total splits).
mi_status check_decode(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* page_table, int32_t pt_stride, const int32_t* ctx_lens,
                       int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                       int64_t num_phys_pages, int32_t num_splits, mi_dtype kv_dtype,
                       const float* o_part, const float* lse_part, DecodeShape* shp,
                       int64_t part_rows = 0) {
  if (!q || !k_cache || !v_cache || !page_table || !ctx_lens || !o_part || !lse_part)
    return MI_ERR_NULL;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || page_size <= 0 || pt_stride <= 0 ||
      num_phys_pages <= 0 || num_splits <= 0 || Hq % Hkv != 0)
    return MI_ERR_SHAPE;
  if (kv_dtype != MI_F16 && kv_dtype != MI_BF16) return MI_ERR_DTYPE;
  const int G = Hq / Hkv;
  if (D != 128 || page_size != 16 || !(G == 1 || G == 2 || G == 4 || G == 8) ||
      num_splits > 1024 || B > 65535 || Hkv > 65535)
    return MI_ERR_UNSUPPORTED;
  if (!size_ok(num_phys_pages, Hkv, static_cast<int64_t>(page_size) * D, 2) ||
      !size_ok(B, Hq, num_splits, D * 4) || !size_ok(B, pt_stride, 4))
    return MI_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(o_part, 16) || !aligned(lse_part, 4) || !aligned(page_table, 4) ||
      !aligned(ctx_lens, 4))
    return MI_ERR_UNSUPPORTED;
  shp->q_bytes = int64_t(B) * Hq * D * 2;
  shp->cache_bytes = num_phys_pages * Hkv * page_size * D * 2;
  shp->pt_bytes = int64_t(B) * pt_stride * 4;
  shp->ctx_bytes = int64_t(B) * 4;
  if (part_rows == 0) part_rows = int64_t(B) * num_splits;
  if (!size_ok(part_rows, Hq, D * 4)) return MI_ERR_SHAPE;
  shp->opart_bytes = part_rows * Hq * D * 4;
  shp->lpart_bytes = part_rows * Hq * 4;
  const void* ins[5] = {q, k_cache, v_cache, page_table, ctx_lens};
  const int64_t in_bytes[5] = {shp->q_bytes, shp->cache_bytes, shp->cache_bytes, shp->pt_bytes,
                               shp->ctx_bytes};
  for (int i = 0; i < 5; ++i) {
    if (overlaps(o_part, shp->opart_bytes, ins[i], in_bytes[i]) ||
        overlaps(lse_part, shp->lpart_bytes, ins[i], in_bytes[i]))
      return MI_ERR_ALIAS;
  }
  if (overlaps(o_part, shp->opart_bytes, lse_part, shp->lpart_bytes)) return MI_ERR_ALIAS;
  return MI_OK;
}

}  // namespace

extern "C" {

const char* mi_status_string(mi_status status) {
  switch (status) {
    case MI_OK: return "MI_OK";
    case MI_ERR_NULL: return "MI_ERR_NULL: a required pointer is NULL";
    case MI_ERR_SHAPE: return "MI_ERR_SHAPE: invalid or inconsistent size";
    case MI_ERR_DTYPE: return "MI_ERR_DTYPE: dtype not allowed for this argument";
    case MI_ERR_UNSUPPORTED: return "MI_ERR_UNSUPPORTED: size, dtype or alignment not supported";
    case MI_ERR_HIP: return "MI_ERR_HIP: a HIP call failed";
    case MI_ERR_ALIAS: return "MI_ERR_ALIAS: outputs overlap inputs";
    case MI_ERR_SCRATCH:
      return "MI_ERR_SCRATCH: more partial rows than the static scratch holds "
             "(B * Hq * num_splits > MI_NOALLOC_MAX_PARTIAL_ROWS)";
  }
  return "unknown mi_status";
}

mi_status mi_merge_state(const void* v_a, const float* s_a, const void* v_b, const float* s_b,
                         void* v_out, float* s_out, int64_t S, int32_t H, int32_t D,
                         mi_dtype v_dtype, mi_dtype out_dtype, void* stream) {
  if (!v_a || !s_a || !v_b || !s_b || !v_out) return MI_ERR_NULL;
  if (S < 0) return MI_ERR_SHAPE;
  mi_status st = check_merge_dims(H, D, v_dtype, out_dtype);
  if (st != MI_OK) return st;
  if (!size_ok(S, H, D, 4)) return MI_ERR_SHAPE;
  if (!aligned(v_a, 16) || !aligned(v_b, 16) || !aligned(v_out, 16) || !aligned(s_a, 4) ||
      !aligned(s_b, 4) || !aligned(s_out, 4))
    return MI_ERR_UNSUPPORTED;
  const int64_t rows = S * H;
  const int64_t in_b = rows * D * dtype_bytes(v_dtype);
  const int64_t out_b = rows * D * dtype_bytes(out_dtype);
  const int64_t s_b_bytes = rows * 4;
  const bool same_dt = v_dtype == out_dtype;
  if (bad_alias(v_out, out_b, v_a, in_b, same_dt) || bad_alias(v_out, out_b, v_b, in_b, same_dt) ||
      overlaps(v_out, out_b, s_a, s_b_bytes) || overlaps(v_out, out_b, s_b, s_b_bytes) ||
      bad_alias(s_out, s_b_bytes, s_a, s_b_bytes, true) ||
      bad_alias(s_out, s_b_bytes, s_b, s_b_bytes, true) ||
      overlaps(s_out, s_b_bytes, v_a, in_b) || overlaps(s_out, s_b_bytes, v_b, in_b) ||
      overlaps(s_out, s_b_bytes, v_out, out_b))
    return MI_ERR_ALIAS;
  if (rows == 0) return MI_OK;
  return from_hip(mi::launch_merge_state(v_a, s_a, v_b, s_b, v_out, s_out, rows, D, v_dtype,
                                         out_dtype, static_cast<hipStream_t>(stream)));
}

mi_status mi_merge_states(const void* v, const float* s, void* v_out, float* s_out, int64_t S,
                          int32_t N, int32_t H, int32_t D, mi_dtype v_dtype, mi_dtype out_dtype,
                          void* stream) {
  if (!v || !s || !v_out) return MI_ERR_NULL;
  if (S < 0 || N <= 0) return MI_ERR_SHAPE;
  mi_status st = check_merge_dims(H, D, v_dtype, out_dtype);
  if (st != MI_OK) return st;
  if (!size_ok(S, N, H, static_cast<int64_t>(D) * 4)) return MI_ERR_SHAPE;
  if (!aligned(v, 16) || !aligned(v_out, 16) || !aligned(s, 4) || !aligned(s_out, 4))
    return MI_ERR_UNSUPPORTED;
  const int64_t in_v = S * N * H * D * dtype_bytes(v_dtype);
  const int64_t in_s = S * N * H * 4;
  const int64_t out_v = S * H * D * dtype_bytes(out_dtype);
  const int64_t out_s = S * H * 4;
  if (overlaps(v_out, out_v, v, in_v) || overlaps(v_out, out_v, s, in_s) ||
      overlaps(s_out, out_s, v, in_v) || overlaps(s_out, out_s, s, in_s) ||
      overlaps(s_out, out_s, v_out, out_v))
    return MI_ERR_ALIAS;
  if (S == 0) return MI_OK;
  return from_hip(mi::launch_merge_states(v, s, v_out, s_out, S, N, H, D, v_dtype, out_dtype,
                                          static_cast<hipStream_t>(stream)));
}

mi_status mi_split_range(int32_t ctx, int32_t page_size, int32_t num_splits, int32_t split,
                         int32_t* p_start, int32_t* p_end) {
  if (!p_start || !p_end) return MI_ERR_NULL;
  if (ctx < 0 || page_size <= 0 || num_splits <= 0 || split < 0 || split >= num_splits)
    return MI_ERR_SHAPE;
  int a, b;
  mi::split_pages(ctx, page_size, num_splits, split, &a, &b);
  *p_start = a;
  *p_end = b;
  return MI_OK;
}

mi_status mi_plan_splits(int32_t B, int32_t Hkv, const int32_t* ctx_lens_host, int32_t page_size,
                         int32_t num_cus, int32_t* num_splits_out) {
  if (!ctx_lens_host || !num_splits_out) return MI_ERR_NULL;
  if (B <= 0 || Hkv <= 0 || page_size <= 0) return MI_ERR_SHAPE;
  int max_pages = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (ctx_lens_host[b] < 0) return MI_ERR_SHAPE;
    const int np = mi::ceil_div(ctx_lens_host[b], page_size);
    if (np > max_pages) max_pages = np;
  }
  if (num_cus <= 0 && device_cus(&num_cus) != MI_OK) return MI_ERR_HIP;
  // "L3 hints", section 6: enough workgroups to fill the device a few times
  // over (here: twice the compute units), but no split thinner than 8 pages.
  static const int kChoices[4] = {1, 4, 16, 64};
  int pick = 3;
  for (int i = 0; i < 4; ++i) {
    if (int64_t(B) * Hkv * kChoices[i] >= 2 * int64_t(num_cus)) {
      pick = i;
      break;
    }
  }
  while (pick > 0 && mi::ceil_div(max_pages, kChoices[pick]) < 8) --pick;
  *num_splits_out = kChoices[pick];
  return MI_OK;
}

mi_status mi_split_kv_partial(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* page_table, int32_t pt_stride,
                              const int32_t* ctx_lens, int32_t B, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t page_size, int64_t num_phys_pages,
                              int32_t num_splits, float sm_scale, mi_dtype kv_dtype,
                              float* o_part, float* lse_part, void* stream) {
  DecodeShape shp;
  mi_status st = check_decode(q, k_cache, v_cache, page_table, pt_stride, ctx_lens, B, Hq, Hkv, D,
                              page_size, num_phys_pages, num_splits, kv_dtype, o_part, lse_part,
                              &shp);
  if (st != MI_OK) return st;
  if (B == 0) return MI_OK;
  return from_hip(mi::launch_split_kv_partial(q, k_cache, v_cache, page_table, pt_stride, ctx_lens,
                                              B, Hq, Hkv, num_phys_pages, num_splits, sm_scale,
                                              kv_dtype, o_part, lse_part,
                                              static_cast<hipStream_t>(stream)));
}

namespace {

// Shared by the two-launch and the fused decode: validation of the outputs
// (and of the counters workspace when it is used).
mi_status check_decode_outputs(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* page_table, const int32_t* ctx_lens,
                               const float* o_part, const float* lse_part,
                               const int32_t* counters, bool need_counters, const void* o,
                               const float* lse, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                               mi_dtype out_dtype, const DecodeShape& shp) {
  if (!o || (need_counters && !counters)) return MI_ERR_NULL;
  if (!dtype_ok(out_dtype)) return MI_ERR_DTYPE;
  if (!aligned(o, 16) || !aligned(lse, 4) || !aligned(counters, 4)) return MI_ERR_UNSUPPORTED;
  const int64_t o_bytes = int64_t(B) * Hq * D * dtype_bytes(out_dtype);
  const int64_t lse_bytes = int64_t(B) * Hq * 4;
  const int64_t cnt_bytes = need_counters ? int64_t(B) * Hkv * 4 : 0;
  const void* all[7] = {q, k_cache, v_cache, page_table, ctx_lens, o_part, lse_part};
  const int64_t all_b[7] = {shp.q_bytes, shp.cache_bytes, shp.cache_bytes, shp.pt_bytes,
                            shp.ctx_bytes, shp.opart_bytes, shp.lpart_bytes};
  for (int i = 0; i < 7; ++i)
    if (overlaps(o, o_bytes, all[i], all_b[i]) || overlaps(lse, lse_bytes, all[i], all_b[i]) ||
        overlaps(counters, cnt_bytes, all[i], all_b[i]))
      return MI_ERR_ALIAS;
  if (overlaps(o, o_bytes, lse, lse_bytes) || overlaps(counters, cnt_bytes, o, o_bytes) ||
      overlaps(counters, cnt_bytes, lse, lse_bytes))
    return MI_ERR_ALIAS;
  return MI_OK;
}

}  // namespace

mi_status mi_split_kv_decode(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* page_table, int32_t pt_stride, const int32_t* ctx_lens,
                             int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                             int64_t num_phys_pages, int32_t num_splits, float sm_scale,
                             mi_dtype kv_dtype, float* o_part, float* lse_part, void* o,
                             float* lse, mi_dtype out_dtype, void* stream) {
  if (!o) return MI_ERR_NULL;
  DecodeShape shp;
  mi_status st = check_decode(q, k_cache, v_cache, page_table, pt_stride, ctx_lens, B, Hq, Hkv, D,
                              page_size, num_phys_pages, num_splits, kv_dtype, o_part, lse_part,
                              &shp);
  if (st != MI_OK) return st;
  st = check_decode_outputs(q, k_cache, v_cache, page_table, ctx_lens, o_part, lse_part, nullptr,
                            false, o, lse, B, Hq, Hkv, D, out_dtype, shp);
  if (st != MI_OK) return st;
  if (B == 0) return MI_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (num_splits == 1)  // one split: pass 1 writes o and lse itself, no combine launch
    return from_hip(mi::launch_split_kv_partial(q, k_cache, v_cache, page_table, pt_stride,
                                                ctx_lens, B, Hq, Hkv, num_phys_pages, 1, sm_scale,
                                                kv_dtype, o_part, lse_part, s, nullptr, o, lse,
                                                out_dtype));
  hipError_t e = mi::launch_split_kv_partial(q, k_cache, v_cache, page_table, pt_stride, ctx_lens,
                                             B, Hq, Hkv, num_phys_pages, num_splits, sm_scale,
                                             kv_dtype, o_part, lse_part, s);
  if (e != hipSuccess) return from_hip(e);
  // The combine: o_part [B, Hq, splits, D] is merge_states' [S = B*Hq, N = splits, H = 1, D].
  return from_hip(mi::launch_merge_states(o_part, lse_part, o, lse, int64_t(B) * Hq, num_splits,
                                          1, D, MI_F32, out_dtype, s));
}

mi_status mi_split_kv_decode_fused(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* page_table, int32_t pt_stride,
                                   const int32_t* ctx_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                   int32_t D, int32_t page_size, int64_t num_phys_pages,
                                   int32_t num_splits, float sm_scale, mi_dtype kv_dtype,
                                   float* o_part, float* lse_part, int32_t* counters, void* o,
                                   float* lse, mi_dtype out_dtype, void* stream) {
  if (!o || !counters) return MI_ERR_NULL;
  DecodeShape shp;
  mi_status st = check_decode(q, k_cache, v_cache, page_table, pt_stride, ctx_lens, B, Hq, Hkv, D,
                              page_size, num_phys_pages, num_splits, kv_dtype, o_part, lse_part,
                              &shp);
  if (st != MI_OK) return st;
  st = check_decode_outputs(q, k_cache, v_cache, page_table, ctx_lens, o_part, lse_part, counters,
                            true, o, lse, B, Hq, Hkv, D, out_dtype, shp);
  if (st != MI_OK) return st;
  if (B == 0) return MI_OK;
  int cus = 0;
  if (device_cus(&cus) != MI_OK) return MI_ERR_HIP;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (num_splits > 1 && !single_launch_pays(int64_t(B) * Hkv * num_splits, cus)) {
    hipError_t e = mi::launch_split_kv_partial(q, k_cache, v_cache, page_table, pt_stride,
                                               ctx_lens, B, Hq, Hkv, num_phys_pages, num_splits,
                                               sm_scale, kv_dtype, o_part, lse_part, hs);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(mi::launch_merge_states(o_part, lse_part, o, lse, int64_t(B) * Hq, num_splits,
                                            1, D, MI_F32, out_dtype, hs));
  }
  return from_hip(mi::launch_split_kv_partial(q, k_cache, v_cache, page_table, pt_stride,
                                              ctx_lens, B, Hq, Hkv, num_phys_pages, num_splits,
                                              sm_scale, kv_dtype, o_part, lse_part, hs, counters,
                                              o, lse, out_dtype));
}

mi_status mi_merge_states_workspace(int64_t S, int32_t N, int32_t H, int32_t D,
                                   size_t* ws_bytes) {
  if (!ws_bytes) return MI_ERR_NULL;
  if (S < 0 || N <= 0 || H <= 0 || D <= 0) return MI_ERR_SHAPE;
  const int parts = mi::merge_states_parts(S, N, H);
  *ws_bytes = parts == 1 ? 0 : static_cast<size_t>(S) * parts * H * (D + 1) * sizeof(float);
  return MI_OK;
}

mi_status mi_merge_states_two_level(const void* v, const float* s, void* v_out, float* s_out,
                                    int64_t S, int32_t N, int32_t H, int32_t D,
                                    mi_dtype v_dtype, mi_dtype out_dtype, float* workspace,
                                    size_t ws_bytes, void* stream) {
  if (!v || !s || !v_out) return MI_ERR_NULL;
  if (S < 0 || N <= 0) return MI_ERR_SHAPE;
  mi_status st = check_merge_dims(H, D, v_dtype, out_dtype);
  if (st != MI_OK) return st;
  if (!size_ok(S, N, H, static_cast<int64_t>(D) * 4)) return MI_ERR_SHAPE;
  size_t need = 0;
  st = mi_merge_states_workspace(S, N, H, D, &need);
  if (st != MI_OK) return st;
  if (need > 0 && !workspace) return MI_ERR_NULL;
  if (ws_bytes < need) return MI_ERR_SHAPE;
  if (!aligned(v, 16) || !aligned(v_out, 16) || !aligned(s, 4) || !aligned(s_out, 4) ||
      !aligned(workspace, 16))
    return MI_ERR_UNSUPPORTED;
  const int64_t in_v = S * N * H * D * dtype_bytes(v_dtype);
  const int64_t in_s = S * N * H * 4;
  const int64_t out_v = S * H * D * dtype_bytes(out_dtype);
  const int64_t out_s = S * H * 4;
  const int64_t ws_b = static_cast<int64_t>(need);
  if (overlaps(v_out, out_v, v, in_v) || overlaps(v_out, out_v, s, in_s) ||
      overlaps(s_out, out_s, v, in_v) || overlaps(s_out, out_s, s, in_s) ||
      overlaps(s_out, out_s, v_out, out_v) || overlaps(workspace, ws_b, v, in_v) ||
      overlaps(workspace, ws_b, s, in_s) || overlaps(workspace, ws_b, v_out, out_v) ||
      overlaps(workspace, ws_b, s_out, out_s))
    return MI_ERR_ALIAS;
  if (S == 0) return MI_OK;
  return from_hip(mi::launch_merge_states_two_level(v, s, v_out, s_out, S, N, H, D, v_dtype,
                                                    out_dtype, workspace,
                                                    static_cast<hipStream_t>(stream)));
}

mi_status mi_merge_state_in_place(void* v, float* s, const void* v_other, const float* s_other,
                                  const uint8_t* mask, int64_t S, int32_t H, int32_t D,
                                  mi_dtype v_dtype, void* stream) {
  if (!v || !s || !v_other || !s_other) return MI_ERR_NULL;
  if (S < 0) return MI_ERR_SHAPE;
  mi_status st = check_merge_dims(H, D, v_dtype, v_dtype);
  if (st != MI_OK) return st;
  if (!size_ok(S, H, D, 4)) return MI_ERR_SHAPE;
  if (!aligned(v, 16) || !aligned(v_other, 16) || !aligned(s, 4) || !aligned(s_other, 4))
    return MI_ERR_UNSUPPORTED;
  const int64_t rows = S * H;
  const int64_t vb = rows * D * dtype_bytes(v_dtype);
  const int64_t sb = rows * 4;
  if (overlaps(v, vb, v_other, vb) || overlaps(v, vb, s_other, sb) || overlaps(v, vb, mask, S) ||
      overlaps(v, vb, s, sb) || overlaps(s, sb, v_other, vb) || overlaps(s, sb, s_other, sb) ||
      overlaps(s, sb, mask, S))
    return MI_ERR_ALIAS;
  if (rows == 0) return MI_OK;
  return from_hip(mi::launch_merge_state_masked(v, s, v_other, s_other, mask, rows, H, D, v_dtype,
                                                static_cast<hipStream_t>(stream)));
}

mi_status mi_merge_sink(const void* v, const float* s, const float* sink, void* v_out,
                        float* s_out, int64_t S, int32_t H, int32_t D, mi_dtype v_dtype,
                        mi_dtype out_dtype, void* stream) {
  if (!v || !s || !sink || !v_out) return MI_ERR_NULL;
  if (S < 0) return MI_ERR_SHAPE;
  mi_status st = check_merge_dims(H, D, v_dtype, out_dtype);
  if (st != MI_OK) return st;
  if (!size_ok(S, H, D, 4)) return MI_ERR_SHAPE;
  if (!aligned(v, 16) || !aligned(v_out, 16) || !aligned(s, 4) || !aligned(s_out, 4) ||
      !aligned(sink, 4))
    return MI_ERR_UNSUPPORTED;
  const int64_t rows = S * H;
  const int64_t in_b = rows * D * dtype_bytes(v_dtype);
  const int64_t out_b = rows * D * dtype_bytes(out_dtype);
  const int64_t sb = rows * 4;
  const int64_t kb = int64_t(H) * 4;
  if (bad_alias(v_out, out_b, v, in_b, v_dtype == out_dtype) || overlaps(v_out, out_b, s, sb) ||
      overlaps(v_out, out_b, sink, kb) || bad_alias(s_out, sb, s, sb, true) ||
      overlaps(s_out, sb, v, in_b) || overlaps(s_out, sb, sink, kb) ||
      overlaps(s_out, sb, v_out, out_b))
    return MI_ERR_ALIAS;
  if (rows == 0) return MI_OK;
  return from_hip(mi::launch_merge_sink(v, s, sink, v_out, s_out, rows, H, D, v_dtype, out_dtype,
                                        static_cast<hipStream_t>(stream)));
}

mi_status mi_merge_states_varlen(const void* v, const float* s, const int32_t* indptr,
                                 int64_t total, void* v_out, float* s_out, int64_t S, int32_t H,
                                 int32_t D, mi_dtype v_dtype, mi_dtype out_dtype, void* stream) {
  if (!v || !s || !indptr || !v_out) return MI_ERR_NULL;
  if (S < 0 || total < 0 || total > INT32_MAX) return MI_ERR_SHAPE;
  mi_status st = check_merge_dims(H, D, v_dtype, out_dtype);
  if (st != MI_OK) return st;
  if (!size_ok(total, H, D, 4) || !size_ok(S, H, D, 4)) return MI_ERR_SHAPE;
  if (!aligned(v, 16) || !aligned(v_out, 16) || !aligned(s, 4) || !aligned(s_out, 4) ||
      !aligned(indptr, 4))
    return MI_ERR_UNSUPPORTED;
  const int64_t in_v = total * H * D * dtype_bytes(v_dtype);
  const int64_t in_s = total * H * 4;
  const int64_t ip = (S + 1) * 4;
  const int64_t out_v = S * H * D * dtype_bytes(out_dtype);
  const int64_t out_s = S * H * 4;
  if (overlaps(v_out, out_v, v, in_v) || overlaps(v_out, out_v, s, in_s) ||
      overlaps(v_out, out_v, indptr, ip) || overlaps(s_out, out_s, v, in_v) ||
      overlaps(s_out, out_s, s, in_s) || overlaps(s_out, out_s, indptr, ip) ||
      overlaps(s_out, out_s, v_out, out_v))
    return MI_ERR_ALIAS;
  if (S == 0) return MI_OK;
  return from_hip(mi::launch_merge_segments(v, s, indptr, total, 0, v_out, s_out, S, H, D, v_dtype,
                                            out_dtype, static_cast<hipStream_t>(stream)));
}

mi_status mi_plan_splits_varlen(int32_t B, int32_t Hkv, const int32_t* ctx_lens_host,
                                int32_t page_size, int32_t num_cus, int32_t* split_indptr_host) {
  if (!ctx_lens_host || !split_indptr_host) return MI_ERR_NULL;
  if (B <= 0 || Hkv <= 0 || page_size <= 0) return MI_ERR_SHAPE;
  int64_t max_np = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (ctx_lens_host[b] < 0) return MI_ERR_SHAPE;
    const int64_t np = (int64_t(ctx_lens_host[b]) + page_size - 1) / page_size;
    if (np > max_np) max_np = np;
  }
  if (num_cus <= 0 && device_cus(&num_cus) != MI_OK) return MI_ERR_HIP;
  // Work items when every split holds at most c pages; never increases with c.
  auto items = [&](int64_t c) {
    int64_t w = 0;
    for (int32_t b = 0; b < B; ++b) {
      const int64_t np = (int64_t(ctx_lens_host[b]) + page_size - 1) / page_size;
      w += np > c ? (np + c - 1) / c : 1;
    }
    return w * Hkv;
  };
  // "L3 hints", section 6, per sequence: the largest page budget c whose work
  // items still reach twice the compute units (the fewest items that fill the
  // device), but at least 8 pages per split. Bisection over [8, max_np].
  const int64_t target = 2 * int64_t(num_cus);
  int64_t c = 8;
  if (max_np > 8 && items(8) >= target) {
    int64_t lo = 8, hi = max_np;  // items(lo) >= target holds throughout
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo + 1) / 2;
      if (items(mid) >= target)
        lo = mid;
      else
        hi = mid - 1;
    }
    c = lo;
  }
  int64_t acc = 0;
  split_indptr_host[0] = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t np = (int64_t(ctx_lens_host[b]) + page_size - 1) / page_size;
    acc += np > c ? (np + c - 1) / c : 1;
    if (acc > INT32_MAX) return MI_ERR_SHAPE;
    split_indptr_host[b + 1] = static_cast<int32_t>(acc);
  }
  return MI_OK;
}

mi_status mi_split_kv_decode_varlen(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* page_table, int32_t pt_stride,
                                    const int32_t* ctx_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                    int32_t D, int32_t page_size, int64_t num_phys_pages,
                                    const int32_t* split_indptr, int32_t total_splits,
                                    float sm_scale, mi_dtype kv_dtype, float* o_part,
                                    float* lse_part, int32_t* counters, void* o, float* lse,
                                    mi_dtype out_dtype, void* stream) {
  if (!o || !split_indptr) return MI_ERR_NULL;
  if (B < 0 || total_splits < 0) return MI_ERR_SHAPE;
  if (B > kMaxVarlenSeqs || total_splits > kMaxVarlenSplits) return MI_ERR_UNSUPPORTED;
  DecodeShape shp;
  mi_status st = check_decode(q, k_cache, v_cache, page_table, pt_stride, ctx_lens, B, Hq, Hkv, D,
                              page_size, num_phys_pages, 1, kv_dtype, o_part, lse_part, &shp,
                              total_splits > 0 ? total_splits : 1);
  if (st != MI_OK) return st;
  st = check_decode_outputs(q, k_cache, v_cache, page_table, ctx_lens, o_part, lse_part, counters,
                            counters != nullptr, o, lse, B, Hq, Hkv, D, out_dtype, shp);
  if (st != MI_OK) return st;
  if (!aligned(split_indptr, 4)) return MI_ERR_UNSUPPORTED;
  const int64_t ip_b = (int64_t(B) + 1) * 4;
  const int64_t o_b = int64_t(B) * Hq * D * dtype_bytes(out_dtype);
  if (overlaps(split_indptr, ip_b, o_part, shp.opart_bytes) ||
      overlaps(split_indptr, ip_b, lse_part, shp.lpart_bytes) ||
      overlaps(split_indptr, ip_b, o, o_b) || overlaps(split_indptr, ip_b, lse, int64_t(B) * Hq * 4) ||
      overlaps(split_indptr, ip_b, counters, counters ? int64_t(B) * Hkv * 4 : 0))
    return MI_ERR_ALIAS;
  if (B == 0) return MI_OK;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (total_splits == 0)  // no work item: every sequence is empty, the combine writes (0, -inf)
    return from_hip(mi::launch_merge_segments(o_part, lse_part, split_indptr, 0, 0, o, lse, B, Hq,
                                              D, MI_F32, out_dtype, hs));
  if (counters != nullptr) {
    int cus = 0;
    if (device_cus(&cus) != MI_OK) return MI_ERR_HIP;
    if (!single_launch_pays(int64_t(total_splits) * Hkv, cus)) counters = nullptr;
  }
  hipError_t e = mi::launch_split_kv_partial_varlen(
      q, k_cache, v_cache, page_table, pt_stride, ctx_lens, B, Hq, Hkv, num_phys_pages,
      split_indptr, total_splits, sm_scale, kv_dtype, o_part, lse_part, hs, counters, o, lse,
      out_dtype);
  if (e != hipSuccess || counters != nullptr) return from_hip(e);
  // The combine: o_part [total, Hq, D] holds sequence b's splits at rows
  // split_indptr[b] .. split_indptr[b+1]-1 -- a segmented merge with H = Hq.
  return from_hip(mi::launch_merge_segments(o_part, lse_part, split_indptr, total_splits, 0, o, lse,
                                            B, Hq, D, MI_F32, out_dtype, hs));
}

mi_status mi_prefix_attention_workspace(int32_t R, int32_t Hq, int32_t Hkv, int32_t D,
                                        int32_t prefix_len, size_t* ws_bytes) {
  if (!ws_bytes) return MI_ERR_NULL;
  if (R < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || prefix_len < 0)
    return MI_ERR_SHAPE;
  if (D != 128) return MI_ERR_UNSUPPORTED;
  int n_chunks, chunk_tokens;
  mi::prefix_attention_plan(R > 0 ? R : 1, Hq, Hkv, prefix_len, &n_chunks, &chunk_tokens);
  *ws_bytes = static_cast<size_t>(R) * Hq * n_chunks * (D + 1) * sizeof(float);
  return MI_OK;
}

mi_status mi_prefix_attention(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* prefix_pages, int32_t prefix_len, int32_t R,
                              int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                              int64_t num_phys_pages, float sm_scale, mi_dtype kv_dtype,
                              float* workspace, size_t ws_bytes, void* v_out, float* s_out,
                              mi_dtype out_dtype, void* stream) {
  if (!q || !k_cache || !v_cache || !workspace || !v_out) return MI_ERR_NULL;
  if (prefix_len > 0 && !prefix_pages) return MI_ERR_NULL;
  if (R < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || page_size <= 0 ||
      prefix_len < 0 || num_phys_pages <= 0)
    return MI_ERR_SHAPE;
  if (kv_dtype != MI_F16 && kv_dtype != MI_BF16) return MI_ERR_DTYPE;
  if (!dtype_ok(out_dtype)) return MI_ERR_DTYPE;
  if (D != 128 || page_size != 16) return MI_ERR_UNSUPPORTED;
  if (!size_ok(num_phys_pages, Hkv, static_cast<int64_t>(page_size) * D, 2) ||
      !size_ok(R, Hq, D, 4))
    return MI_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(workspace, 16) || !aligned(v_out, 16) || !aligned(s_out, 4) ||
      !aligned(prefix_pages, 4))
    return MI_ERR_UNSUPPORTED;
  size_t need = 0;
  mi_status st = mi_prefix_attention_workspace(R, Hq, Hkv, D, prefix_len, &need);
  if (st != MI_OK) return st;
  if (ws_bytes < need) return MI_ERR_SHAPE;
  const int64_t q_b = int64_t(R) * Hq * D * 2;
  const int64_t cache_b = num_phys_pages * Hkv * page_size * D * 2;
  const int64_t pp_b = int64_t(mi::ceil_div(prefix_len, page_size)) * 4;
  const int64_t vo_b = int64_t(R) * Hq * D * dtype_bytes(out_dtype);
  const int64_t so_b = int64_t(R) * Hq * 4;
  const int64_t ws_b = static_cast<int64_t>(need);
  const void* ins[4] = {q, k_cache, v_cache, prefix_pages};
  const int64_t in_b[4] = {q_b, cache_b, cache_b, pp_b};
  for (int i = 0; i < 4; ++i)
    if (overlaps(workspace, ws_b, ins[i], in_b[i]) || overlaps(v_out, vo_b, ins[i], in_b[i]) ||
        overlaps(s_out, so_b, ins[i], in_b[i]))
      return MI_ERR_ALIAS;
  if (overlaps(workspace, ws_b, v_out, vo_b) || overlaps(workspace, ws_b, s_out, so_b) ||
      overlaps(v_out, vo_b, s_out, so_b))
    return MI_ERR_ALIAS;
  if (R == 0) return MI_OK;
  int n_chunks, chunk_tokens;
  mi::prefix_attention_plan(R, Hq, Hkv, prefix_len, &n_chunks, &chunk_tokens);
  float* ws_o = workspace;
  float* ws_s = workspace + static_cast<int64_t>(R) * Hq * n_chunks * D;
  return from_hip(mi::launch_prefix_attention(q, k_cache, v_cache, prefix_pages, prefix_len, R,
                                              Hq, Hkv, num_phys_pages, sm_scale, kv_dtype, ws_o,
                                              ws_s, v_out, s_out, out_dtype,
                                              static_cast<hipStream_t>(stream)));
}

mi_status mi_cascade_decode(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* prefix_pages, int32_t prefix_len,
                            const int32_t* suffix_table, int32_t suffix_stride,
                            const int32_t* suffix_lens, int32_t R, int32_t Hq, int32_t Hkv,
                            int32_t D, int32_t page_size, int64_t num_phys_pages,
                            int32_t suffix_splits, float sm_scale, mi_dtype kv_dtype,
                            float* workspace, size_t ws_bytes, float* o_part, float* lse_part,
                            int32_t* counters, void* o, float* lse, mi_dtype out_dtype,
                            void* stream) {
  if (!o || !counters || !workspace) return MI_ERR_NULL;
  if (prefix_len > 0 && !prefix_pages) return MI_ERR_NULL;
  if (prefix_len < 0) return MI_ERR_SHAPE;
  DecodeShape shp;
  mi_status st = check_decode(q, k_cache, v_cache, suffix_table, suffix_stride, suffix_lens, R,
                              Hq, Hkv, D, page_size, num_phys_pages, suffix_splits, kv_dtype,
                              o_part, lse_part, &shp);
  if (st != MI_OK) return st;
  st = check_decode_outputs(q, k_cache, v_cache, suffix_table, suffix_lens, o_part, lse_part,
                            counters, true, o, lse, R, Hq, Hkv, D, out_dtype, shp);
  if (st != MI_OK) return st;
  size_t need = 0;
  st = mi_prefix_attention_workspace(R, Hq, Hkv, D, prefix_len, &need);
  if (st != MI_OK) return st;
  if (ws_bytes < need) return MI_ERR_SHAPE;
  if (!aligned(workspace, 16) || !aligned(prefix_pages, 4)) return MI_ERR_UNSUPPORTED;
  const int64_t ws_b = static_cast<int64_t>(need);
  const int64_t pp_b = int64_t(mi::ceil_div(prefix_len, page_size)) * 4;
  const int64_t o_b = int64_t(R) * Hq * D * dtype_bytes(out_dtype);
  const void* all[10] = {q, k_cache, v_cache, suffix_table, suffix_lens, o_part, lse_part,
                         counters, o, lse};
  const int64_t all_b[10] = {shp.q_bytes, shp.cache_bytes, shp.cache_bytes, shp.pt_bytes,
                             shp.ctx_bytes, shp.opart_bytes, shp.lpart_bytes,
                             int64_t(R) * Hkv * 4, o_b, int64_t(R) * Hq * 4};
  for (int i = 0; i < 10; ++i)
    if (overlaps(workspace, ws_b, all[i], all_b[i]) || overlaps(prefix_pages, pp_b, all[i], all_b[i]))
      return MI_ERR_ALIAS;
  if (overlaps(workspace, ws_b, prefix_pages, pp_b)) return MI_ERR_ALIAS;
  if (R == 0) return MI_OK;
  int n_chunks, chunk_tokens;
  mi::prefix_attention_plan(R, Hq, Hkv, prefix_len, &n_chunks, &chunk_tokens);
  float* ws_o = workspace;
  float* ws_s = workspace + static_cast<int64_t>(R) * Hq * n_chunks * D;
  return from_hip(mi::launch_cascade_decode(
      q, k_cache, v_cache, prefix_pages, prefix_len, suffix_table, suffix_stride, suffix_lens, R,
      Hq, Hkv, num_phys_pages, suffix_splits, sm_scale, kv_dtype, ws_o, ws_s, o_part, lse_part,
      counters, o, lse, out_dtype, static_cast<hipStream_t>(stream)));
}

mi_status mi_stream_read(const void* x, int64_t bytes, uint32_t* xor_out, void* stream) {
  if (bytes < 0 || bytes % 16 != 0) return MI_ERR_SHAPE;
  if (bytes == 0) return MI_OK;
  if (!x || !xor_out) return MI_ERR_NULL;
  if (!aligned(x, 16) || !aligned(xor_out, 4)) return MI_ERR_UNSUPPORTED;
  if (overlaps(xor_out, 4, x, bytes)) return MI_ERR_ALIAS;
  return from_hip(mi::launch_stream_read(x, bytes, xor_out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
