// Split-KV paged decode, pass 1, for gfx950 ("L3 hints: split-KV decode and
// LSE merge", sections 1-5; Flash-Decoding's producer).
//
// One workgroup per (split, kv head, sequence). The split's pages come from
// the page-range formula; each page of the paged cache holds, per kv head, a
// contiguous [PAGE=16, D=128] tile (4 KiB in fp16/bf16).
//
// Work mapping inside the workgroup (4 waves, 256 lanes):
//  - wave w owns token slots 4w..4w+3 of every page; within a wave, lane l
//    owns slot 4w + l/16 and the 8-element chunk (l%16)*8 of D. A wave's
//    quarter of a K or V tile is one contiguous KiB, read with a single fully
//    coalesced 16-byte-per-lane load.
//  - all G = Hq/Hkv query heads of the kv head are served from the same loaded
//    tile (GQA reuse): q.k partial dots use v_dot2 (fp16/bf16 pairs into fp32),
//    and a 16-lane DPP reduction completes each score.
//  - every 16-lane row is its own online-softmax stream (m, l, acc) in base 2:
//    the softmax scale is multiplied by log2(e) once on the host, so weights
//    are the hardware exp2. Streams are merged at the end with the state merge
//    (wave-internal cross-lane, then across waves through LDS).
//  - pages are software-pipelined: each wave keeps kDepth pages of K and V in
//    flight in registers while it computes on earlier ones; the physical page
//    ids come from the page table through the scalar cache.
//
// Guards: the running max is replaced by 0 when it is -inf before it is
// subtracted ("FlashAttention's empty-row LSE", section 2.3), so fully masked
// streams never form -inf - (-inf). Token slots at or past ctx are excluded by
// select on both the score and the value, so whatever they hold (even NaN)
// cannot leak. An empty split writes o = 0 and lse = -inf ("L3 hints",
// section 4).
#include "common.h"
#include "launch.h"
#include "split_range.h"

#include <type_traits>

namespace mi {
namespace {

constexpr int kD = 128;
constexpr int kPage = 16;
// Pages in flight per wave, and page groups per workgroup (4 waves each).
#ifndef MI_DECODE_DEPTH
#define MI_DECODE_DEPTH 4
#endif
#ifndef MI_DECODE_PAGE_GROUPS
#define MI_DECODE_PAGE_GROUPS 1
#endif
constexpr int kDepth = MI_DECODE_DEPTH;
constexpr int kPageGroups = MI_DECODE_PAGE_GROUPS;
constexpr int kWaves = 4 * kPageGroups;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleSlack = 8.0f;
// Word 3 of a gfx9 buffer descriptor for raw (untyped, unswizzled) access.
constexpr int kBufferFlags = 0x00020000;
// Cache policy of the K/V loads (bit 1: non-temporal / streaming).
#ifndef MI_DECODE_KV_POLICY
#define MI_DECODE_KV_POLICY 2
#endif
constexpr int kKvCachePolicy = MI_DECODE_KV_POLICY;
// s_waitcnt immediate (gfx9 encoding) for vmcnt(0), other counters unconstrained.
constexpr int kWaitVmcnt0 = 0x0F70;

template <int DT>
__device__ __forceinline__ float dot8(const u32x4_t& q, const u32x4_t& k) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (DT == MI_F16)
      acc = __builtin_amdgcn_fdot2(as_half2(q[i]), as_half2(k[i]), acc, false);
    else
      acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(q[i]), as_bf162(k[i]), acc, false);
  }
  return acc;
}

template <int DT>
__device__ __forceinline__ void unpack8(const u32x4_t& w, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (DT == MI_F16) {
      x[2 * i] = f16_lo(w[i]);
      x[2 * i + 1] = f16_hi(w[i]);
    } else {
      x[2 * i] = bf16_lo(w[i]);
      x[2 * i + 1] = bf16_hi(w[i]);
    }
  }
}

// The combine of one (sequence, query head) row by one wave: merge the
// `count` partial states of that row ("L3 hints: split-KV decode and LSE
// merge", section 3), and `prior_n` earlier states of the row if given, into
// o[row, :] (dtype DTO) and lse[row] (base 2, optional). Split j's state is
// lse_part[first + j * stride] and o_part[(first + j * stride) * D, ...]:
// stride 1 for the uniform layout [B, Hq, splits], Hq for the per-sequence
// layout [total, Hq]. Earlier state i is prior_s[row * prior_n + i] and
// prior_o[(row * prior_n + i) * D, ...] (a cascade's prefix chunk states).
// Lane l owns the 8-element chunk (l%16)*8 of D for the states j = l/16
// (mod 4); each pass keeps 8 of its states' loads in flight, then the four
// sub-groups are merged across lanes.
template <int DTO>
__device__ void combine_row(const float* o_part, const float* lse_part, int64_t first,
                            int64_t stride, int count, const float* prior_o,
                            const float* prior_s, int prior_n, int64_t row, void* o, float* lse,
                            int lane) {
  const int c = lane & 15;
  const int sg = lane >> 4;
  const int n_all = prior_n + count;
  float m = -kInf, z = 0.0f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  for (int k0 = sg; k0 < n_all; k0 += 32) {
    float sv[8], x[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      int k = k0 + 4 * u;
      k = k < n_all ? k : 0;
      const bool pre = k < prior_n;
      const int64_t r = pre ? row * prior_n + k : first + static_cast<int64_t>(k - prior_n) * stride;
      sv[u] = (pre ? prior_s : lse_part)[r];
      load8<MI_F32>(pre ? prior_o : o_part, r * kD + c * 8, x[u]);
    }
    float cm = m;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      sv[u] = k0 + 4 * u < n_all ? sanitize_lse(sv[u]) : -kInf;
      cm = __builtin_fmaxf(cm, sv[u]);
    }
    const float keep = guarded_exp2(m - cm);
    z *= keep;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= keep;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = guarded_exp2(sv[u] - cm);
      z += w;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = (w > 0.0f) ? __builtin_fmaf(w, x[u][e], acc[e]) : acc[e];
    }
    m = cm;
  }
#pragma unroll
  for (int sh = 16; sh <= 32; sh <<= 1) {
    const float mo = shfl_xor(m, sh);
    const float zo = shfl_xor(z, sh);
    const float M = __builtin_fmaxf(m, mo);
    const float ws = guarded_exp2(m - M);
    const float wo = guarded_exp2(mo - M);
    z = z * ws + zo * wo;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] * ws + shfl_xor(acc[e], sh) * wo;
    m = M;
  }
  if (sg == 0) {
    const float inv = guarded_inv(z);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = acc[e] * inv;
    store8<DTO>(o, row * kD + c * 8, y);
    if (lse != nullptr && c == 0) lse[row] = (z > 0.0f) ? m + hw_log2(z) : -kInf;
  }
}

// Per-sequence splits: the sequence b that owns work item `item`, i.e. the b
// with indptr[b] <= item < indptr[b+1], and that range. Two rounds of a 64-way
// search by the whole wave: lane j first reads indptr at j * stride
// (stride = ceil((B+1)/64) <= 63), the ballot of entries <= item brackets b to
// one stride, and a second read of that bracket finds it. Empty segments are
// skipped by construction (the last entry <= item wins). Results are clamped
// to valid ranges whatever the device data holds: b in [0, B), and
// 0 <= first <= end <= total.
__device__ __forceinline__ void find_segment(const int32_t* indptr, int B, int item, int total,
                                             int* b_out, int* first, int* end) {
  const int lane = __lane_id();
  const int stride = (B + 64) / 64;
  auto probe = [&](int base, int step, int* jl, int* val) {
    int j = base + lane * step;
    j = j < B ? j : B;
    *val = indptr[j];
    const uint64_t below = __builtin_amdgcn_ballot_w64(*val <= item);
    const int cnt = __builtin_popcountll(below);
    *jl = cnt > 0 ? cnt - 1 : 0;
  };
  int jl, val;
  probe(0, stride, &jl, &val);
  int base = 0;
  if (stride > 1) {
    base = jl * stride;
    probe(base, 1, &jl, &val);
  }
  int b = base + jl;
  int lo = __builtin_amdgcn_readlane(val, jl);
  int hi = __builtin_amdgcn_readlane(val, jl < 63 ? jl + 1 : 63);
  b = b < B ? b : B - 1;
  lo = lo < 0 ? 0 : (lo > total ? total : lo);
  hi = hi < lo ? lo : (hi > total ? total : hi);
  *b_out = b;
  *first = lo;
  *end = hi;
}

// DTO < 0: pass 1 only. DTO = an output dtype: pass 1 fused with the combine
// (the last workgroup of each (sequence, kv head) to finish merges the splits).
// kVar: per-sequence split counts. blockIdx.y is then a work item of the
// index pointer array split_indptr [B+1] (sequence b owns items
// split_indptr[b] .. split_indptr[b+1]-1, item k of it being split k of that
// many), and the partials are laid out [total items, Hq, D] / [total, Hq].
// Otherwise blockIdx.y is the split and blockIdx.z the sequence, and the
// partials are [B, Hq, num_splits, D] / [B, Hq, num_splits].
// prior_n > 0 (fused form only): the combine also merges prior_n earlier
// states per (sequence, query head) row, prior_o [rows, prior_n, D] and
// prior_s [rows, prior_n] -- the shared-prefix states of a cascade.
// kPR > 0 (fused, one split per sequence, G <= 4, at most kPR prior states):
// each wave loads its head's prior states (two columns per lane) into
// registers at the start, so the merge at the end needs no memory round trip.
template <int DT, int G, int DTO, bool kVar, int kPR>
__global__ __launch_bounds__(kThreads) void split_kv_partial_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ page_table, int pt_stride,
    const int32_t* __restrict__ ctx_lens, int Hkv, int64_t num_phys, int num_splits,
    float qk_scale_log2, float* __restrict__ o_part, float* __restrict__ lse_part,
    int32_t* __restrict__ counters, void* __restrict__ o, float* __restrict__ lse,
    const int32_t* __restrict__ split_indptr, int B, const float* __restrict__ prior_o,
    const float* __restrict__ prior_s, int prior_n) {
  __shared__ float lds_acc[kWaves][G][kD];
  __shared__ float lds_ml[kWaves][G][2];

  // blockIdx.x is the kv head: consecutive workgroups go round-robin to the
  // XCDs, so each kv head's splits stay on one XCD (and its L2).
  const int hkv = blockIdx.x;
  int b, split, nsplit;  // sequence, split within it, its number of splits
  int seg_first = 0;     // kVar: the sequence's first work item
  if constexpr (kVar) {
    const int item = blockIdx.y;
    int seg_end;
    find_segment(split_indptr, B, item, static_cast<int>(gridDim.y), &b, &seg_first, &seg_end);
    b = __builtin_amdgcn_readfirstlane(b);
    seg_first = __builtin_amdgcn_readfirstlane(seg_first);
    nsplit = __builtin_amdgcn_readfirstlane(seg_end - seg_first);
    split = item - seg_first;
  } else {
    split = blockIdx.y;
    b = blockIdx.z;
    nsplit = num_splits;
  }
  // The wave index is uniform across the wave: readfirstlane tells the
  // compiler so (it keeps wave-derived values in scalar registers).
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int pg = wave >> 2;          // page group: pages pg, pg + kPageGroups, ...
  const int quarter = wave & 3;      // token slots 4*quarter .. 4*quarter+3 of a page
  const int slot = quarter * 4 + (lane >> 4);
  const int d0 = (lane & 15) * 8;
  const int Hq = Hkv * G;

  // Device lengths are clamped: negative -> 0, at most pt_stride pages.
  int64_t ctx64 = ctx_lens[b];
  ctx64 = ctx64 < 0 ? 0 : ctx64;
  const int64_t cap = static_cast<int64_t>(pt_stride) * kPage;
  const int ctx = static_cast<int>(ctx64 < cap ? ctx64 : cap);
  int p0 = 0, p1 = 0;
  // (kVar with inconsistent device data: an item outside its sequence's range
  // attends to nothing.)
  if (split >= 0 && split < nsplit) split_pages(ctx, kPage, nsplit, split, &p0, &p1);
  const int npages = p1 > p0 ? p1 - p0 : 0;

  u32x4_t qw[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qw[h] = *reinterpret_cast<const u32x4_t*>(q + (static_cast<int64_t>(b) * Hq + hkv * G + h) * kD + d0);

  constexpr int kPRg = G <= kWaves ? kPR : 0;  // one head per wave
  float2 pri_o[kPRg > 0 ? kPRg : 1];
  float pri_s[kPRg > 0 ? kPRg : 1];
  if constexpr (kPRg > 0) {
    const int hw = wave < G ? wave : 0;
    const int64_t r0 = (static_cast<int64_t>(b) * Hq + hkv * G + hw) * prior_n;
#pragma unroll
    for (int i = 0; i < kPRg; ++i) {
      const int64_t r = r0 + (i < prior_n ? i : 0);
      pri_s[i] = prior_s[r];
      pri_o[i] = *reinterpret_cast<const float2*>(prior_o + r * kD + 2 * lane);
    }
  }

  // m[h] is the reference max, mu[h] the value subtracted before exp2 (m, or
  // 0 while m is -inf), thr[h] = m + kRescaleSlack; mu and thr change only
  // when m does.
  float m[G], mu[G], thr[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -kInf;
    mu[h] = 0.0f;
    thr[h] = -kInf;
    l[h] = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[h][j] = 0.0f;
  }

  // Page ids: lane l holds the id of page (c0 + l) of the split for the chunk
  // starting at page c0; issues broadcast them with readlane.
  const int32_t* pt = page_table + static_cast<int64_t>(b) * pt_stride + p0;
  auto load_ids = [&](int first) {
    const int i = first + lane;
    return pt[i < npages ? i : npages - 1];
  };

  // Each page's K and V tiles for this kv head are read through a buffer
  // descriptor covering exactly that 4 KiB tile. Pages past the split's end,
  // and page ids outside [0, num_phys), get a descriptor with no records: the
  // hardware returns zeros for them without touching memory, so every
  // prefetch below is unconditional.
  const int lane_bytes = (quarter * 64 + lane) * 16;
  const int64_t tile_elems = static_cast<int64_t>(kPage) * kD;
  u32x4_t kb[kDepth], vb[kDepth];
  bool ok[kDepth];
  int ids = 0;
  // issue(k, n, j): the wave's k-th page of the current chunk (chunk-relative
  // page r = pg + k*kPageGroups of n) into register slot j.
  auto issue = [&](int k, int n, int j) {
    const int r = pg + k * kPageGroups;
    const int32_t phys = __builtin_amdgcn_readlane(ids, r & 63);
    ok[j] = r < n && phys >= 0 && phys < num_phys;
    const int64_t tile = (static_cast<int64_t>(ok[j] ? phys : 0) * Hkv + hkv) * tile_elems;
    const int records = ok[j] ? static_cast<int>(tile_elems * 2) : 0;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kc + tile), 0, records, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vc + tile), 0, records, kBufferFlags);
    kb[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, lane_bytes, 0, kKvCachePolicy));
    vb[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, lane_bytes, 0, kKvCachePolicy));
  };

  // Online softmax with a lazily updated reference max m[h]: exponentials are
  // taken against m[h] and the accumulators are rescaled only when a score
  // exceeds m[h] by more than kRescaleSlack (or on a stream's first token), so
  // p <= 2^kRescaleSlack and the common step is one exp2 and 8 FMAs per head.
  // The state (m, l, acc) stays exact: l and acc are always relative to m.
  auto consume = [&](int i, int j, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    const bool valid = !kMasked || ((p0 + i) * kPage + slot < ctx);
    const bool page_ok = ok[j];  // false: past the split or a bad page id (zeros were loaded)
    float v[8];
    unpack8<DT>(vb[j], v);
    if constexpr (kMasked) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = valid ? v[e] : 0.0f;
    }
    // The G partial dots are reduced over the 16 lanes of a row step by step
    // for all heads together, so the DPP steps of different heads interleave
    // (a DPP read of a just-written VGPR otherwise needs wait states).
    float x[G];
#pragma unroll
    for (int h = 0; h < G; ++h) x[h] = dot8<DT>(qw[h], kb[j]);
#pragma unroll
    for (int h = 0; h < G; ++h) x[h] += dpp<kDppQuadXor1>(x[h]);
#pragma unroll
    for (int h = 0; h < G; ++h) x[h] += dpp<kDppQuadXor2>(x[h]);
#pragma unroll
    for (int h = 0; h < G; ++h) x[h] += dpp<kDppRowRor4>(x[h]);
#pragma unroll
    for (int h = 0; h < G; ++h) x[h] += dpp<kDppRowRor8>(x[h]);
    bool need_any = false;
    bool need[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      x[h] = (valid && page_ok) ? x[h] * qk_scale_log2 : -kInf;
      need[h] = x[h] > thr[h];
      need_any |= need[h];
    }
    if (__builtin_amdgcn_ballot_w64(need_any) != 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float alpha = need[h] ? __builtin_amdgcn_exp2f(m[h] - x[h]) : 1.0f;
        m[h] = need[h] ? x[h] : m[h];
        mu[h] = (m[h] == -kInf) ? 0.0f : m[h];
        thr[h] = m[h] + kRescaleSlack;
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p = __builtin_amdgcn_exp2f(x[h] - mu[h]);
      l[h] += p;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = __builtin_fmaf(p, v[e], acc[h][e]);
    }
  };
  // The only page that can hold slots at or past ctx is the sequence's last
  // page when ctx is not a multiple of the page size. If this split holds it,
  // it is taken out of the pipelined loop (which then needs no masking) and
  // handled once at the end with the masked step.
  const bool has_tail = npages > 0 && (ctx % kPage) != 0 && p1 - 1 == ctx / kPage;
  const int nmain = npages - (has_tail ? 1 : 0);

  // Pages are processed in chunks of 64 (one VGPR of page ids per chunk).
  // Within a chunk the loop body holds only the K/V loads, each slot being
  // re-issued right after it is consumed; the scheduling barrier keeps that
  // order so every consume waits only for the load issued kDepth pages earlier.
  for (int c0 = 0; c0 < nmain; c0 += 64) {
    const int n = nmain - c0 < 64 ? nmain - c0 : 64;
    const int n_local = n > pg ? (n - pg + kPageGroups - 1) / kPageGroups : 0;
    ids = load_ids(c0);
#pragma unroll
    for (int j = 0; j < kDepth; ++j) {
      issue(j, n, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int iters = (n_local + kDepth - 1) / kDepth * kDepth;
    for (int base = 0; base < iters; base += kDepth) {
#pragma unroll
      for (int j = 0; j < kDepth; ++j) {
        consume(c0 + pg + (base + j) * kPageGroups, j, std::false_type{});
        issue(base + j + kDepth, n, j);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (has_tail && nmain % kPageGroups == pg) {
    ids = load_ids(nmain & ~63);
    issue((nmain & 63) / kPageGroups, (nmain & 63) + 1, 0);
    consume(nmain, 0, std::true_type{});
  }

  // Merge the four token rows of the wave (lanes l, l^16, l^32, l^48).
#pragma unroll
  for (int sh = 16; sh <= 32; sh <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = shfl_xor(m[h], sh);
      const float lo = shfl_xor(l[h], sh);
      const float M = __builtin_fmaxf(m[h], mo);
      const float ws = guarded_exp2(m[h] - M);
      const float wo = guarded_exp2(mo - M);
      l[h] = l[h] * ws + lo * wo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ao = shfl_xor(acc[h][e], sh);
        acc[h][e] = acc[h][e] * ws + ao * wo;
      }
      m[h] = M;
    }
  }

  // Merge the waves through LDS; wave w finalises heads w, w+4, ...
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) lds_acc[wave][h][d0 + e] = acc[h][e];
      if (lane == 0) {
        lds_ml[wave][h][0] = m[h];
        lds_ml[wave][h][1] = l[h];
      }
    }
  }
  __syncthreads();
  for (int h = wave; h < G; h += kWaves) {
    float M = -kInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = __builtin_fmaxf(M, lds_ml[w][h][0]);
    float Z = 0.0f, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float ww = guarded_exp2(lds_ml[w][h][0] - M);
      Z = __builtin_fmaf(ww, lds_ml[w][h][1], Z);
      o0 = __builtin_fmaf(ww, lds_acc[w][h][2 * lane], o0);
      o1 = __builtin_fmaf(ww, lds_acc[w][h][2 * lane + 1], o1);
    }
    const float inv = guarded_inv(Z);
    const int64_t row = static_cast<int64_t>(b) * Hq + hkv * G + h;
    // This split's partial row: [B, Hq, splits] or [total, Hq].
    const int64_t prow = kVar ? static_cast<int64_t>(blockIdx.y) * Hq + hkv * G + h
                              : row * num_splits + split;
    float* out = o_part + prow * kD + 2 * lane;
    const float2 res = make_float2(o0 * inv, o1 * inv);
    const float lse_val = (Z > 0.0f) ? M + hw_log2(Z) : -kInf;
    if constexpr (DTO >= 0 && kPRg > 0) {
      // The only split: merge with this row's prior states held in registers.
      *reinterpret_cast<float2*>(out) = res;
      if (lane == 0) lse_part[prow] = lse_val;
      float ps[kPRg];
      float mx = lse_val;
#pragma unroll
      for (int i = 0; i < kPRg; ++i) {
        ps[i] = i < prior_n ? sanitize_lse(pri_s[i]) : -kInf;
        mx = __builtin_fmaxf(mx, ps[i]);
      }
      const float w0 = guarded_exp2(lse_val - mx);
      float z = w0;
      float a0 = w0 > 0.0f ? w0 * res.x : 0.0f;
      float a1 = w0 > 0.0f ? w0 * res.y : 0.0f;
#pragma unroll
      for (int i = 0; i < kPRg; ++i) {
        const float w = guarded_exp2(ps[i] - mx);
        z += w;
        a0 = w > 0.0f ? __builtin_fmaf(w, pri_o[i].x, a0) : a0;
        a1 = w > 0.0f ? __builtin_fmaf(w, pri_o[i].y, a1) : a1;
      }
      const float zi = guarded_inv(z);
      const float2 fin = make_float2(a0 * zi, a1 * zi);
      if constexpr (DTO == MI_F32) {
        *reinterpret_cast<float2*>(static_cast<float*>(o) + row * kD + 2 * lane) = fin;
      } else {
        const uint32_t w2 = DTO == MI_F16 ? pack_f16(fin.x, fin.y) : pack_bf16(fin.x, fin.y);
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(o) + row * kD + 2 * lane) = w2;
      }
      if (lse != nullptr && lane == 0) lse[row] = (z > 0.0f) ? mx + hw_log2(z) : -kInf;
      continue;
    }
    if constexpr (DTO >= 0) {
      if (nsplit == 1 && prior_n == 0) {
        // One split: the combine is the identity, so write the result directly.
        *reinterpret_cast<float2*>(out) = res;
        if (lane == 0) lse_part[prow] = lse_val;
        if constexpr (DTO == MI_F32) {
          *reinterpret_cast<float2*>(static_cast<float*>(o) + row * kD + 2 * lane) = res;
        } else {
          const uint32_t w2 = DTO == MI_F16 ? pack_f16(res.x, res.y) : pack_bf16(res.x, res.y);
          *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(o) + row * kD + 2 * lane) = w2;
        }
        if (lse != nullptr && lane == 0) lse[row] = lse_val;
        continue;
      }
      // Agent-scope stores are written through to the device coherence point,
      // so another XCD can read them without a writeback of this XCD's L2.
      __hip_atomic_store(reinterpret_cast<uint64_t*>(out), __builtin_bit_cast(uint64_t, res),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0)
        __hip_atomic_store(lse_part + prow, lse_val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      *reinterpret_cast<float2*>(out) = res;
      if (lane == 0) lse_part[prow] = lse_val;
    }
  }

  if constexpr (DTO >= 0) {
    if (kPRg > 0 || (nsplit == 1 && prior_n == 0)) return;  // written directly above
    if (nsplit == 1) {
      // The only split, with earlier states to merge: this workgroup holds
      // everything it needs, so ordering its own stores before its own loads
      // (workgroup scope) suffices -- no counter, and no device-wide acquire
      // that would drop other workgroups' cached K/V.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __syncthreads();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      for (int h = wave; h < G; h += kWaves) {
        const int64_t row = static_cast<int64_t>(b) * Hq + hkv * G + h;
        const int64_t first = kVar ? static_cast<int64_t>(seg_first) * Hq + hkv * G + h
                                   : row * num_splits;
        combine_row<DTO>(o_part, lse_part, first, 1, 1, prior_o, prior_s, prior_n, row, o, lse,
                         lane);
      }
      return;
    }
    // Hand-off: every workgroup publishes its partials (agent-scope release)
    // and bumps the (sequence, kv head) counter; the one that brings it to
    // num_splits performs the acquire and merges all splits of its heads.
    __shared__ int is_last;
    // Publish: the partials above were written with write-through agent-scope
    // stores; waiting for them to complete (vmcnt(0)) before the barrier and
    // the counter update orders them before it without a whole-L2 writeback.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (threadIdx.x == 0) {
      const int prev = __hip_atomic_fetch_add(counters + static_cast<int64_t>(b) * Hkv + hkv, 1,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      is_last = prev == nsplit - 1;
    }
    __syncthreads();
    if (!is_last) return;
    // Acquire at agent scope: drop stale lines before reading other
    // workgroups' partials.
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    for (int h = wave; h < G; h += kWaves) {
      const int64_t row = static_cast<int64_t>(b) * Hq + hkv * G + h;
      if constexpr (kVar)
        combine_row<DTO>(o_part, lse_part, static_cast<int64_t>(seg_first) * Hq + hkv * G + h, Hq,
                         nsplit, prior_o, prior_s, prior_n, row, o, lse, lane);
      else
        combine_row<DTO>(o_part, lse_part, row * num_splits, 1, nsplit, prior_o, prior_s,
                         prior_n, row, o, lse, lane);
    }
    if (threadIdx.x == 0) counters[static_cast<int64_t>(b) * Hkv + hkv] = 0;
  }
}

template <int DT, int DTO, bool kVar, int kPR = 0>
hipError_t launch_group(int G, dim3 grid, hipStream_t st, const void* q, const void* kc,
                        const void* vc, const int32_t* pt, int pt_stride, const int32_t* ctx,
                        int Hkv, int64_t num_phys, int num_splits, float scale, float* o_part,
                        float* lse_part, int32_t* counters, void* o, float* lse,
                        const int32_t* split_indptr, int B, const float* prior_o,
                        const float* prior_s, int prior_n) {
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(kc);
  const uint16_t* v16 = static_cast<const uint16_t*>(vc);
#define MI_LAUNCH_G(GG)                                                                        \
  split_kv_partial_kernel<DT, GG, DTO, kVar, kPR><<<grid, kThreads, 0, st>>>(                  \
      q16, k16, v16, pt, pt_stride, ctx, Hkv, num_phys, num_splits, scale, o_part, lse_part, \
      counters, o, lse, split_indptr, B, prior_o, prior_s, prior_n)
  switch (G) {
    case 1: MI_LAUNCH_G(1); break;
    case 2: MI_LAUNCH_G(2); break;
    case 4: MI_LAUNCH_G(4); break;
    default: MI_LAUNCH_G(8); break;
  }
#undef MI_LAUNCH_G
  return hipGetLastError();
}

template <int DT, bool kVar>
hipError_t launch_dtype(int out_dtype, int G, dim3 grid, hipStream_t st, const void* q,
                        const void* kc, const void* vc, const int32_t* pt, int pt_stride,
                        const int32_t* ctx, int Hkv, int64_t num_phys, int num_splits, float scale,
                        float* o_part, float* lse_part, int32_t* counters, void* o, float* lse,
                        const int32_t* split_indptr, int B, const float* prior_o = nullptr,
                        const float* prior_s = nullptr, int prior_n = 0) {
  // Prior states in registers: one split, at most 16 of them, one head per wave.
  constexpr int kPR = 16;
  if constexpr (!kVar) {
    if (prior_n > 0 && prior_n <= kPR && num_splits == 1 && G <= 4 && out_dtype >= 0) {
      switch (out_dtype) {
        case MI_F16:
          return launch_group<DT, MI_F16, false, kPR>(G, grid, st, q, kc, vc, pt, pt_stride, ctx, Hkv, num_phys, num_splits, scale, o_part, lse_part, counters, o, lse, split_indptr, B, prior_o, prior_s, prior_n);
        case MI_BF16:
          return launch_group<DT, MI_BF16, false, kPR>(G, grid, st, q, kc, vc, pt, pt_stride, ctx, Hkv, num_phys, num_splits, scale, o_part, lse_part, counters, o, lse, split_indptr, B, prior_o, prior_s, prior_n);
        default:
          return launch_group<DT, MI_F32, false, kPR>(G, grid, st, q, kc, vc, pt, pt_stride, ctx, Hkv, num_phys, num_splits, scale, o_part, lse_part, counters, o, lse, split_indptr, B, prior_o, prior_s, prior_n);
      }
    }
  }
  switch (out_dtype) {
    case MI_F16:
      return launch_group<DT, MI_F16, kVar>(G, grid, st, q, kc, vc, pt, pt_stride, ctx, Hkv, num_phys, num_splits, scale, o_part, lse_part, counters, o, lse, split_indptr, B, prior_o, prior_s, prior_n);
    case MI_BF16:
      return launch_group<DT, MI_BF16, kVar>(G, grid, st, q, kc, vc, pt, pt_stride, ctx, Hkv, num_phys, num_splits, scale, o_part, lse_part, counters, o, lse, split_indptr, B, prior_o, prior_s, prior_n);
    case MI_F32:
      return launch_group<DT, MI_F32, kVar>(G, grid, st, q, kc, vc, pt, pt_stride, ctx, Hkv, num_phys, num_splits, scale, o_part, lse_part, counters, o, lse, split_indptr, B, prior_o, prior_s, prior_n);
    default:
      return launch_group<DT, -1, kVar>(G, grid, st, q, kc, vc, pt, pt_stride, ctx, Hkv, num_phys, num_splits, scale, o_part, lse_part, nullptr, nullptr, nullptr, split_indptr, B, nullptr, nullptr, 0);
  }
}

}  // namespace

hipError_t launch_split_kv_partial(const void* q, const void* kc, const void* vc,
                                   const int32_t* page_table, int pt_stride,
                                   const int32_t* ctx_lens, int B, int Hq, int Hkv,
                                   int64_t num_phys_pages, int num_splits, float sm_scale,
                                   int kv_dtype, float* o_part, float* lse_part,
                                   hipStream_t st, int32_t* counters, void* o, float* lse,
                                   int out_dtype, const float* prior_o, const float* prior_s,
                                   int prior_n) {
  const int G = Hq / Hkv;
  const dim3 grid(static_cast<unsigned>(Hkv), static_cast<unsigned>(num_splits),
                  static_cast<unsigned>(B));
  const float scale = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  // o is written by this kernel when fused (counters given) or when there is a
  // single split (no combine needed); otherwise pass 1 only.
  const int dto = (counters != nullptr || (o != nullptr && num_splits == 1)) ? out_dtype : -1;
  if (kv_dtype == MI_F16)
    return launch_dtype<MI_F16, false>(dto, G, grid, st, q, kc, vc, page_table, pt_stride,
                                       ctx_lens, Hkv, num_phys_pages, num_splits, scale, o_part,
                                       lse_part, counters, o, lse, nullptr, B, prior_o, prior_s,
                                       prior_n);
  return launch_dtype<MI_BF16, false>(dto, G, grid, st, q, kc, vc, page_table, pt_stride,
                                      ctx_lens, Hkv, num_phys_pages, num_splits, scale, o_part,
                                      lse_part, counters, o, lse, nullptr, B, prior_o, prior_s,
                                      prior_n);
}

hipError_t launch_split_kv_partial_varlen(const void* q, const void* kc, const void* vc,
                                          const int32_t* page_table, int pt_stride,
                                          const int32_t* ctx_lens, int B, int Hq, int Hkv,
                                          int64_t num_phys_pages, const int32_t* split_indptr,
                                          int total_splits, float sm_scale, int kv_dtype,
                                          float* o_part, float* lse_part, hipStream_t st,
                                          int32_t* counters, void* o, float* lse, int out_dtype) {
  const int G = Hq / Hkv;
  const dim3 grid(static_cast<unsigned>(Hkv), static_cast<unsigned>(total_splits), 1);
  const float scale = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  const int dto = counters != nullptr ? out_dtype : -1;
  if (kv_dtype == MI_F16)
    return launch_dtype<MI_F16, true>(dto, G, grid, st, q, kc, vc, page_table, pt_stride,
                                      ctx_lens, Hkv, num_phys_pages, 0, scale, o_part, lse_part,
                                      counters, o, lse, split_indptr, B);
  return launch_dtype<MI_BF16, true>(dto, G, grid, st, q, kc, vc, page_table, pt_stride,
                                     ctx_lens, Hkv, num_phys_pages, 0, scale, o_part, lse_part,
                                     counters, o, lse, split_indptr, B);
}

}  // namespace mi
