// Split-KV paged decode, pass 1 and its single-launch combine, for gfx950
// ("L3 hints: split-KV decode and LSE merge", sections 1-5; Flash-Decoding's
// producer).
//
// One workgroup (4 waves) per work item: a (split, kv head, sequence). The
// split's pages come from the page-range formula; each page of the paged
// cache holds, per kv head, a contiguous [PAGE=16, D=128] tile (4 KiB in
// fp16/bf16).
//
// Work mapping:
//  - a wave owns whole pages: wave w takes pages w, w+4, w+8, ... of the
//    split and reads each page's K and V tiles itself, so the four waves never
//    wait for one another inside the loop.
//  - within a wave, a lane serves one token group and one or two 8-element
//    chunks of D (Layout below): with two chunks per lane (G <= 4), 8 lanes
//    cover a token row, so a load instruction reads 8 full 128-byte row
//    halves and each lane holds 2 tokens of the page. Every K or V load is 16
//    bytes per lane.
//  - all G = Hq/Hkv query heads of the kv head use the same loaded tile (GQA
//    reuse): q.k partial dots use v_dot2 (fp16/bf16 pairs into fp32) and a
//    DPP reduction over the row's lanes completes each score.
//  - the online softmax (m, l, acc) runs in base 2: the softmax scale is
//    multiplied by log2(e) once on the host, so weights are the hardware
//    exp2. The reference max m is shared by the whole wave, so the partial
//    sums of its lane groups add without rescaling at the end; the waves'
//    states are merged through LDS with the state merge.
//  - pages are software-pipelined: each wave keeps kDepth pages of K and V in
//    flight in registers while it computes on earlier ones.
//
// Counting instructions per 8 KiB page at G = 4 (fp16): 64 dot2, 24 DPP adds,
// 8 exp2 and 128 fp16-by-fp32 FMAs plus about 40 others -- about 60% of what a
// 16-lanes-per-token mapping needs, which on MI355X keeps the vector units
// below the memory stream instead of ahead of it.
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
// Pages in flight per wave (each page is 8 KiB of K and V for one kv head).
constexpr int kDepth = 2;
constexpr int kWaves = 4;
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
// Ordering of the single-launch hand-off's counter update. 0 (default): a
// relaxed agent-scope add after the write-through partial stores have
// completed; this relies on how gfx942/gfx950 perform agent-scope stores
// (written through to the device coherence point, acknowledged only once
// there). 1: a release add, which the language memory model alone makes
// sufficient, at the cost of an L2 writeback in every workgroup.
#ifndef MI_DECODE_STRICT_RELEASE
#define MI_DECODE_STRICT_RELEASE 0
#endif

template <int DT>
__device__ __forceinline__ float dot8acc(const u32x4_t& q, const u32x4_t& k, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (DT == MI_F16)
      acc = __builtin_amdgcn_fdot2(as_half2(q[i]), as_half2(k[i]), acc, false);
    else
      acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf162(q[i]), as_bf162(k[i]), acc, false);
  }
  return acc;
}

// Lane layout of the decode kernel for G query heads per kv head: each lane
// holds kCpl 8-element chunks of a token row (two for G <= 4, one for G = 8,
// which keeps the G accumulators within the register budget), so kLpt lanes
// cover a row, one load instruction covers kTpi tokens, and a lane holds kTpl
// tokens of each page.
template <int G>
struct Layout {
  static constexpr int kCpl = G <= 4 ? 2 : 1;
  static constexpr int kLpt = 16 / kCpl;
  static constexpr int kTpi = 64 / kLpt;
  static constexpr int kTpl = kPage / kTpi;
};

constexpr int kDppRowHalfMirror = 0x141;  // mirror within each half-row of 8 lanes

// Maximum over the 64 lanes of a wave, returned to every lane.
__device__ __forceinline__ float wave_max(float x) {
  x = __builtin_fmaxf(x, dpp<kDppQuadXor1>(x));
  x = __builtin_fmaxf(x, dpp<kDppQuadXor2>(x));
  x = __builtin_fmaxf(x, dpp<kDppRowRor4>(x));
  x = __builtin_fmaxf(x, dpp<kDppRowRor8>(x));
  const int xi = __builtin_bit_cast(int, x);
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
  return __builtin_fmaxf(__builtin_fmaxf(a, b), __builtin_fmaxf(c, d));
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
// (mod 4); a pass issues the loads of all its (up to kCombineInflight) states
// before using any, then the four sub-groups are merged across lanes.
constexpr int kCombineInflight = 8;
template <int DTO>
__device__ void combine_row(const float* o_part, const float* lse_part, int64_t first,
                            int64_t stride, int count, const float* prior_o,
                            const float* prior_s, int prior_n, int64_t row, void* o, float* lse,
                            int lane) {
  constexpr int U = kCombineInflight;
  const int c = lane & 15;
  const int sg = lane >> 4;
  const int n_all = prior_n + count;
  float m = -kInf, z = 0.0f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  for (int k0 = sg; k0 < n_all; k0 += 4 * U) {
    float sv[U], x[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int k = k0 + 4 * u;
      k = k < n_all ? k : k0;
      const bool pre = k < prior_n;
      const int64_t r = pre ? row * prior_n + k : first + static_cast<int64_t>(k - prior_n) * stride;
      sv[u] = (pre ? prior_s : lse_part)[r];
      load8<MI_F32>(pre ? prior_o : o_part, r * kD + c * 8, x[u]);
    }
    float cm = m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      sv[u] = k0 + 4 * u < n_all ? sanitize_lse(sv[u]) : -kInf;
      cm = __builtin_fmaxf(cm, sv[u]);
    }
    const float keep = guarded_exp2(m - cm);
    z *= keep;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= keep;
#pragma unroll
    for (int u = 0; u < U; ++u) {
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


// Sum over the 64 lanes of a wave, returned to every lane.
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowRor4>(x);
  x += dpp<kDppRowRor8>(x);
  const int xi = __builtin_bit_cast(int, x);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48)));
}

// The combine of one row without prior states, one wave: every load
// instruction reads two whole state rows (lane l: row 2u + l/32 of the pass,
// elements 4*(l%32) .. +3), so the wave's reads are contiguous 1 KiB blocks
// in the uniform layout. Lane l also loads the LSE of state l of the pass;
// the pass maximum and the weights come from wave reductions, and each
// lane takes the weights of its rows with readlane. A pass covers 2U states
// with all their loads in flight at once.
template <int DTO, int U>
__device__ void combine_row_wide(const float* o_part, const float* lse_part, int64_t first,
                                 int stride, int count, int64_t row, void* o, float* lse,
                                 int lane) {
  const int half = lane >> 5;
  const int c4 = (lane & 31) * 4;
  float M = -kInf, Z = 0.0f, acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = 0; k0 < count; k0 += 2 * U) {
    const int kl = k0 + lane;
    float sl = -kInf;
    if (lane < 2 * U && kl < count) sl = sanitize_lse(lse_part[first + static_cast<int64_t>(kl) * stride]);
    float4_t x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int ku = k0 + 2 * u + half;
      ku = ku < count ? ku : k0;
      x[u] = __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(
          o_part + (first + static_cast<int64_t>(ku) * stride) * kD + c4));
    }
    const float Mn = __builtin_fmaxf(M, wave_max(sl));
    const float keep = guarded_exp2(M - Mn);
    Z *= keep;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= keep;
    M = Mn;
    const float w = guarded_exp2(sl - M);
    Z += wave_sum(w);
    const int wi = __builtin_bit_cast(int, w);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(wi, 2 * u));
      const float w1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(wi, 2 * u + 1));
      const float wu = half ? w1 : w0;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = (wu > 0.0f) ? __builtin_fmaf(wu, x[u][e], acc[e]) : acc[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] += shfl_xor(acc[e], 32);
  if (half == 0) {
    const float inv = guarded_inv(Z);
    const float y0 = acc[0] * inv, y1 = acc[1] * inv, y2 = acc[2] * inv, y3 = acc[3] * inv;
    if constexpr (DTO == MI_F32) {
      *reinterpret_cast<float4_t*>(static_cast<float*>(o) + row * kD + c4) = float4_t{y0, y1, y2, y3};
    } else {
      const uint32_t a = DTO == MI_F16 ? pack_f16(y0, y1) : pack_bf16(y0, y1);
      const uint32_t b2 = DTO == MI_F16 ? pack_f16(y2, y3) : pack_bf16(y2, y3);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(o) + row * kD + c4) = make_uint2(a, b2);
    }
    if (lse != nullptr && lane == 0) lse[row] = (Z > 0.0f) ? M + hw_log2(Z) : -kInf;
  }
}

// The combine of one row: the register-lean form when there are no prior
// states and the offsets fit, the general one otherwise.
template <int DTO>
__device__ __forceinline__ void combine_any(const float* o_part, const float* lse_part,
                                            int64_t first, int64_t stride, int count,
                                            const float* prior_o, const float* prior_s,
                                            int prior_n, int64_t row, void* o, float* lse,
                                            int lane) {
  if (prior_n == 0 && static_cast<int64_t>(count) * stride * kD * 4 < (int64_t(1) << 31)) {
    const int st = static_cast<int>(stride);
    if (count <= 4)
      combine_row_wide<DTO, 2>(o_part, lse_part, first, st, count, row, o, lse, lane);
    else if (count <= 16)
      combine_row_wide<DTO, 8>(o_part, lse_part, first, st, count, row, o, lse, lane);
    else
      combine_row_wide<DTO, 32>(o_part, lse_part, first, st, count, row, o, lse, lane);
    return;
  }
  combine_row<DTO>(o_part, lse_part, first, stride, count, prior_o, prior_s, prior_n, row, o, lse,
                   lane);
}

// Writes the empty state (o = 0, lse = -inf) of the G query-head rows of kv
// head hkv of sequence b; one wave, lane l owning two elements.
template <int DTO, int G>
__device__ __forceinline__ void write_empty_rows(int b, int Hq, int hkv, void* o, float* lse,
                                                 int lane) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int64_t row = static_cast<int64_t>(b) * Hq + hkv * G + h;
    if constexpr (DTO == MI_F32)
      *reinterpret_cast<float2*>(static_cast<float*>(o) + row * kD + 2 * lane) = make_float2(0.0f, 0.0f);
    else
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(o) + row * kD + 2 * lane) = 0u;
    if (lse != nullptr && lane == 0) lse[row] = -kInf;
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

// One workgroup per work item of one kv head. Work item j is, in the uniform
// layout, split j % num_splits of sequence j / num_splits (partials
// [B, Hq, num_splits, D] / [B, Hq, num_splits]); with kVar, it is item j of
// the index pointer array split_indptr [B+1] (sequence b owns items
// split_indptr[b] .. split_indptr[b+1]-1, item k of it being split k of that
// many; partials [total, Hq, D] / [total, Hq]). blockIdx.x = hkv + Hkv * j,
// so consecutive workgroups are a kv head's neighbours: the dispatcher deals
// workgroups round-robin to the XCDs, so with 8 kv heads every split of a kv
// head runs on one XCD and shares its L2 for the page table and q.
// DTO < 0: pass 1 only. DTO = an output dtype: pass 1 fused with the combine
// (the last item of each (sequence, kv head) to finish merges the splits).
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
    const float* __restrict__ prior_s, int prior_n, int total_items) {
  __shared__ float lds_part[kWaves][4][G][kD];
  __shared__ float lds_l[kWaves][4][G];
  __shared__ float lds_m[kWaves][G];
  __shared__ int lds_go;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int quarter = wave;  // the wave's pages: quarter, quarter + 4, ... of the split
  const int Hq = Hkv * G;
  const int hkv = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x % Hkv));
  const int item = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x / Hkv));
  // b: the sequence; split: this item's split of it; nsplit: that sequence's
  // split count; in_range: the item is one of its sequence's splits.
  const bool has_row = item < total_items;
  int b = 0, split = 0, nsplit = 1, seg_first = 0, seg_end = 0;
  bool in_range = has_row;
  if (has_row) {
    if constexpr (kVar) {
      find_segment(split_indptr, B, item, total_items, &b, &seg_first, &seg_end);
      b = __builtin_amdgcn_readfirstlane(b);
      seg_first = __builtin_amdgcn_readfirstlane(seg_first);
      seg_end = __builtin_amdgcn_readfirstlane(seg_end);
      nsplit = seg_end - seg_first;
      split = item - seg_first;
      // (inconsistent device data: an item outside its sequence's range
      // attends to nothing, writes an empty partial and takes no part in a
      // combine)
      in_range = split >= 0 && split < nsplit;
    } else {
      b = item / num_splits;
      split = item - b * num_splits;
      nsplit = num_splits;
    }
  }
  // The split-0 item of a sequence also writes the empty state of sequences
  // with no split: the ones right before it, and all after it when it is the
  // last sequence with splits. Entries read now, used at the end.
  int prev_entry = -1, last_entry = -1;
  if constexpr (kVar && DTO >= 0) {
    if (in_range && split == 0) {
      prev_entry = b > 0 ? split_indptr[b - 1] : -1;
      last_entry = split_indptr[B];
    }
  }

  // Speculative page ids (uniform layout): before the sequence length
  // arrives, assume a full page-table row (pt_stride pages) and fetch the
  // first chunk's ids of that guess, so that the id load is not queued behind
  // the length load. Used only if the guess gives the real first page.
  int spec_p0 = -1, spec_ids = 0;
  if constexpr (!kVar) {
    if (in_range) {
      spec_p0 = split * ceil_div(pt_stride, nsplit);
      const int i = spec_p0 + lane;
      spec_ids = page_table[static_cast<int64_t>(b) * pt_stride + (i < pt_stride ? i : pt_stride - 1)];
    }
  }
  // Device lengths are clamped: negative -> 0, at most pt_stride pages.
  int64_t ctx64 = ctx_lens[b];
  ctx64 = ctx64 < 0 ? 0 : ctx64;
  const int64_t cap = static_cast<int64_t>(pt_stride) * kPage;
  const int ctx = static_cast<int>(ctx64 < cap ? ctx64 : cap);
  int p0 = 0, p1 = 0;
  if (in_range) split_pages(ctx, kPage, nsplit, split, &p0, &p1);
  const int npages = p1 > p0 ? p1 - p0 : 0;

  // Lane mapping (a wave owns whole pages): lane l serves the token group
  // g = l / kLpt, i.e. tokens g + kTpi*j (j < kTpl) of every page it reads,
  // and the 8-element chunks c + kLpt*k (k < kCpl) of D, c = l % kLpt. One
  // 16-byte load of the K or V tile per (j, k) and lane: the kLpt lanes of a
  // group read 16 * kLpt contiguous bytes of a token row per instruction.
  using Lay = Layout<G>;
  constexpr int kCpl = Lay::kCpl, kLpt = Lay::kLpt, kTpi = Lay::kTpi, kTpl = Lay::kTpl;
  const int tg = lane / kLpt;
  const int ch = lane % kLpt;
  const int row16 = lane >> 4;

  u32x4_t qw[G][kCpl];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int k = 0; k < kCpl; ++k)
      qw[h][k] = *reinterpret_cast<const u32x4_t*>(
          q + (static_cast<int64_t>(b) * Hq + hkv * G + h) * kD + 8 * (ch + kLpt * k));

  constexpr int kPRg = G <= 4 ? kPR : 0;  // one head per wave of the item
  float2 pri_o[kPRg > 0 ? kPRg : 1];
  float pri_s[kPRg > 0 ? kPRg : 1];
  if constexpr (kPRg > 0) {
    const int hw = quarter < G ? quarter : 0;
    const int64_t r0 = (static_cast<int64_t>(b) * Hq + hkv * G + hw) * prior_n;
#pragma unroll
    for (int i = 0; i < kPRg; ++i) {
      const int64_t r = r0 + (i < prior_n ? i : 0);
      pri_s[i] = prior_s[r];
      pri_o[i] = *reinterpret_cast<const float2*>(prior_o + r * kD + 2 * lane);
    }
  }

  // The wave's reference max m[h] is uniform across the wave (so the
  // streams of its lane groups add up without rescaling at the end); mu[h] is
  // the value subtracted before exp2 (m, or 0 while m is -inf) and thr[h] =
  // m + kRescaleSlack. l[h] and acc are per lane group, relative to m[h].
  float m[G], mu[G], thr[G], l[G], acc[G][kCpl][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -kInf;
    mu[h] = 0.0f;
    thr[h] = -kInf;
    l[h] = 0.0f;
#pragma unroll
    for (int k = 0; k < kCpl; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][k][e] = 0.0f;
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
  // prefetch below is unconditional (and their consume is skipped).
  const int lane_bytes = tg * (kD * 2) + 16 * ch;
  const int64_t tile_elems = static_cast<int64_t>(kPage) * kD;
  u32x4_t kb[kDepth][kTpl][kCpl], vb[kDepth][kTpl][kCpl];
  bool ok[kDepth];
  int ids = 0;
  // issue(r, n, s): page r of the current chunk (of n pages) into register slot s.
  auto issue = [&](int r, int n, int s) {
    const int32_t phys = __builtin_amdgcn_readlane(ids, r & 63);
    ok[s] = r < n && phys >= 0 && phys < num_phys;
    const int64_t tile = (static_cast<int64_t>(ok[s] ? phys : 0) * Hkv + hkv) * tile_elems;
    const int records = ok[s] ? static_cast<int>(tile_elems * 2) : 0;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kc + tile), 0, records, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vc + tile), 0, records, kBufferFlags);
#pragma unroll
    for (int j = 0; j < kTpl; ++j)
#pragma unroll
      for (int k = 0; k < kCpl; ++k) {
        const int off = lane_bytes + j * kTpi * (kD * 2) + k * kLpt * 16;
        kb[s][j][k] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, kKvCachePolicy));
      }
#pragma unroll
    for (int j = 0; j < kTpl; ++j)
#pragma unroll
      for (int k = 0; k < kCpl; ++k) {
        const int off = lane_bytes + j * kTpi * (kD * 2) + k * kLpt * 16;
        vb[s][j][k] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kKvCachePolicy));
      }
  };

  // One page (in slot s) of the online softmax. The reference max moves only
  // when a score exceeds it by more than kRescaleSlack (or on the first
  // token), so p <= 2^kRescaleSlack and the common step is one exp2 per
  // token and head plus the V FMAs. The state stays exact: l and acc are
  // always relative to m.
  auto consume = [&](int i, int s, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    bool valid[kTpl];
#pragma unroll
    for (int j = 0; j < kTpl; ++j) valid[j] = !kMasked || ((p0 + i) * kPage + tg + kTpi * j < ctx);
    float x[kTpl][G];
#pragma unroll
    for (int j = 0; j < kTpl; ++j)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.0f;
#pragma unroll
        for (int k = 0; k < kCpl; ++k) a = dot8acc<DT>(qw[h][k], kb[s][j][k], a);
        x[j][h] = a;
      }
    // Sum over the kLpt lanes of a group, step by step for every (token,
    // head) together so no DPP read waits on the VGPR it just wrote.
#pragma unroll
    for (int j = 0; j < kTpl; ++j)
#pragma unroll
      for (int h = 0; h < G; ++h) x[j][h] += dpp<kDppQuadXor1>(x[j][h]);
#pragma unroll
    for (int j = 0; j < kTpl; ++j)
#pragma unroll
      for (int h = 0; h < G; ++h) x[j][h] += dpp<kDppQuadXor2>(x[j][h]);
    if constexpr (kLpt == 8) {
#pragma unroll
      for (int j = 0; j < kTpl; ++j)
#pragma unroll
        for (int h = 0; h < G; ++h) x[j][h] += dpp<kDppRowHalfMirror>(x[j][h]);
    } else {
#pragma unroll
      for (int j = 0; j < kTpl; ++j)
#pragma unroll
        for (int h = 0; h < G; ++h) x[j][h] += dpp<kDppRowRor4>(x[j][h]);
#pragma unroll
      for (int j = 0; j < kTpl; ++j)
#pragma unroll
        for (int h = 0; h < G; ++h) x[j][h] += dpp<kDppRowRor8>(x[j][h]);
    }
    bool need_any = false;
    float xm[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      xm[h] = -kInf;
#pragma unroll
      for (int j = 0; j < kTpl; ++j) {
        x[j][h] = valid[j] ? x[j][h] * qk_scale_log2 : -kInf;
        xm[h] = __builtin_fmaxf(xm[h], x[j][h]);
      }
      need_any |= xm[h] > thr[h];
    }
    if (__builtin_amdgcn_ballot_w64(need_any) != 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float M = wave_max(xm[h]);
        if (M > thr[h]) {
          const float alpha = __builtin_amdgcn_exp2f(m[h] - M);
          m[h] = M;
          mu[h] = M;
          thr[h] = M + kRescaleSlack;
          l[h] *= alpha;
#pragma unroll
          for (int k = 0; k < kCpl; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][k][e] *= alpha;
        }
      }
    }
    float v[kTpl][kCpl][8];
#pragma unroll
    for (int j = 0; j < kTpl; ++j)
#pragma unroll
      for (int k = 0; k < kCpl; ++k) {
        u32x4_t w = vb[s][j][k];
        if constexpr (kMasked) {
#pragma unroll
          for (int d = 0; d < 4; ++d) w[d] = valid[j] ? w[d] : 0u;
        }
        unpack8<DT>(w, v[j][k]);
      }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < kTpl; ++j) {
        const float p = __builtin_amdgcn_exp2f(x[j][h] - mu[h]);
        l[h] += p;
#pragma unroll
        for (int k = 0; k < kCpl; ++k)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][k][e] = __builtin_fmaf(p, v[j][k][e], acc[h][k][e]);
      }
  };
  // The only page that can hold slots at or past ctx is the sequence's last
  // page when ctx is not a multiple of the page size. If this split holds it,
  // it is taken out of the pipelined loop (which then needs no masking) and
  // handled once at the end with the masked step.
  const bool has_tail = npages > 0 && (ctx % kPage) != 0 && p1 - 1 == ctx / kPage;
  const int nmain = npages - (has_tail ? 1 : 0);

  // Pages are processed in chunks of 64 (one VGPR of page ids per chunk);
  // wave `quarter` of the item takes pages quarter, quarter + 4, ... of each
  // chunk. The loop body holds only the K/V loads, each slot being re-issued
  // right after it is consumed; the scheduling barrier keeps that order so
  // every consume waits only for the load issued kDepth pages earlier.
  for (int c0 = 0; c0 < nmain; c0 += 64) {
    const int n = nmain - c0 < 64 ? nmain - c0 : 64;
    const int n_local = n > quarter ? (n - quarter + 3) / 4 : 0;
    ids = (c0 == 0 && spec_p0 == p0) ? spec_ids : load_ids(c0);
#pragma unroll
    for (int s = 0; s < kDepth; ++s) {
      issue(quarter + 4 * s, n, s);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int iters = (n_local + kDepth - 1) / kDepth * kDepth;
    for (int base = 0; base < iters; base += kDepth) {
#pragma unroll
      for (int s = 0; s < kDepth; ++s) {
        if (ok[s]) consume(c0 + quarter + 4 * (base + s), s, std::false_type{});
        issue(quarter + 4 * (base + s + kDepth), n, s);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (has_tail && (nmain & 3) == quarter) {
    ids = load_ids(nmain & ~63);
    issue(nmain & 63, (nmain & 63) + 1, 0);
    if (ok[0]) consume(nmain, 0, std::true_type{});
  }

  // The wave's lane groups share m, so their states add: first the two groups
  // of a 16-lane row (kLpt = 8), then the rows and waves through LDS.
  if constexpr (kLpt == 8) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      l[h] += dpp<kDppRowRor8>(l[h]);
#pragma unroll
      for (int k = 0; k < kCpl; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][k][e] += dpp<kDppRowRor8>(acc[h][k][e]);
    }
  }
  if ((lane & 15) < kLpt) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int k = 0; k < kCpl; ++k) {
        float* dst = &lds_part[wave][row16][h][8 * (ch + kLpt * k)];
        *reinterpret_cast<float4_t*>(dst) = float4_t{acc[h][k][0], acc[h][k][1], acc[h][k][2], acc[h][k][3]};
        *reinterpret_cast<float4_t*>(dst + 4) = float4_t{acc[h][k][4], acc[h][k][5], acc[h][k][6], acc[h][k][7]};
      }
      if (ch == 0) lds_l[wave][row16][h] = l[h];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) lds_m[wave][h] = m[h];
  }
  __syncthreads();
  // What follows pass 1 for this item (fused form): 0 nothing (no item, the
  // combine was the identity, or the item is outside its sequence), 1 a local
  // merge with prior states (the only split: this workgroup holds everything
  // it needs), 2 the counter hand-off.
  const int mode = (DTO < 0 || !in_range || kPRg > 0 || (nsplit == 1 && prior_n == 0)) ? 0
                   : (nsplit == 1 ? 1 : 2);
  for (int h = quarter; h < G && has_row; h += 4) {
    float M = -kInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = __builtin_fmaxf(M, lds_m[w][h]);
    float Z = 0.0f, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float ww = guarded_exp2(lds_m[w][h] - M);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float2 pv = *reinterpret_cast<const float2*>(&lds_part[w][r][h][2 * lane]);
        Z = __builtin_fmaf(ww, lds_l[w][r][h], Z);
        o0 = __builtin_fmaf(ww, pv.x, o0);
        o1 = __builtin_fmaf(ww, pv.y, o1);
      }
    }
    const float inv = guarded_inv(Z);
    const int64_t row = static_cast<int64_t>(b) * Hq + hkv * G + h;
    // This item's partial row: [B, Hq, splits] or [total, Hq].
    const int64_t prow = kVar ? static_cast<int64_t>(item) * Hq + hkv * G + h
                              : row * num_splits + split;
    float* out = o_part + prow * kD + 2 * lane;
    const float2 res = make_float2(o0 * inv, o1 * inv);
    const float lse_val = (Z > 0.0f) ? M + hw_log2(Z) : -kInf;
    if (mode == 2) {
      // Agent-scope stores are written through to the device coherence
      // point, so another XCD can read them without a writeback of this
      // XCD's L2.
      __hip_atomic_store(reinterpret_cast<uint64_t*>(out), __builtin_bit_cast(uint64_t, res),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0)
        __hip_atomic_store(lse_part + prow, lse_val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      continue;
    }
    *reinterpret_cast<float2*>(out) = res;
    if (lane == 0) lse_part[prow] = lse_val;
    if constexpr (DTO >= 0) {
      if (!in_range) continue;
      if constexpr (kPRg > 0) {
        // The only split: merge with this row's prior states held in registers.
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
      } else if (nsplit == 1 && prior_n == 0) {
        // One split: the combine is the identity, so write the result directly.
        if constexpr (DTO == MI_F32) {
          *reinterpret_cast<float2*>(static_cast<float*>(o) + row * kD + 2 * lane) = res;
        } else {
          const uint32_t w2 = DTO == MI_F16 ? pack_f16(res.x, res.y) : pack_bf16(res.x, res.y);
          *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(o) + row * kD + 2 * lane) = w2;
        }
        if (lse != nullptr && lane == 0) lse[row] = lse_val;
      }
    }
  }

  if constexpr (DTO >= 0) {
    // Hand-off. Mode 2: every item publishes its partials and bumps the
    // (sequence, kv head) counter; the one that brings it to nsplit performs
    // the acquire and merges all splits of its heads. Publish: the partials
    // above were written with write-through agent-scope stores; waiting for
    // them to complete (vmcnt(0)) before the barrier and the counter update
    // orders them before it without a whole-L2 writeback. Mode 1: workgroup
    // scope suffices -- no counter, and no device-wide acquire that would drop
    // other workgroups' cached K/V.
    if (mode == 2) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (mode == 1) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (quarter == 0 && lane == 0) {
      int go = mode == 1 ? 1 : 0;
      if (mode == 2) {
        const int prev = __hip_atomic_fetch_add(
            counters + static_cast<int64_t>(b) * Hkv + hkv, 1,
            MI_DECODE_STRICT_RELEASE ? __ATOMIC_RELEASE : __ATOMIC_RELAXED,
            __HIP_MEMORY_SCOPE_AGENT);
        go = prev == nsplit - 1 ? 2 : 0;
      }
      lds_go = go;
    }
    __syncthreads();
    const int go = __builtin_amdgcn_readfirstlane(lds_go);
    if (go == 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // Acquire at agent scope: drop stale lines before reading other
    // workgroups' partials.
    if (go == 2) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (go != 0) {
      for (int h = quarter; h < G; h += 4) {
        const int64_t row = static_cast<int64_t>(b) * Hq + hkv * G + h;
        if constexpr (kVar)
          combine_any<DTO>(o_part, lse_part, static_cast<int64_t>(seg_first) * Hq + hkv * G + h, Hq,
                           nsplit, prior_o, prior_s, prior_n, row, o, lse, lane);
        else
          combine_any<DTO>(o_part, lse_part, row * num_splits, 1, nsplit, prior_o, prior_s,
                           prior_n, row, o, lse, lane);
      }
      if (go == 2 && quarter == 0 && lane == 0) counters[static_cast<int64_t>(b) * Hkv + hkv] = 0;
    }
    if constexpr (kVar) {
      // Sequences with no split get the empty state (0, -inf).
      if (quarter == 0 && prev_entry == seg_first && b > 0) {
        for (int bb = b - 1; bb >= 0; --bb) {
          if (split_indptr[bb] != seg_first) break;
          write_empty_rows<DTO, G>(bb, Hq, hkv, o, lse, lane);
        }
      }
      if (quarter == 0 && last_entry == seg_end && in_range && split == 0) {
        for (int bb = b + 1; bb < B; ++bb) write_empty_rows<DTO, G>(bb, Hq, hkv, o, lse, lane);
      }
    }
  }
}

template <int DT, int DTO, bool kVar, int kPR = 0>
hipError_t launch_group(int G, unsigned blocks, hipStream_t st, const void* q, const void* kc,
                        const void* vc, const int32_t* pt, int pt_stride, const int32_t* ctx,
                        int Hkv, int64_t num_phys, int num_splits, float scale, float* o_part,
                        float* lse_part, int32_t* counters, void* o, float* lse,
                        const int32_t* split_indptr, int B, const float* prior_o,
                        const float* prior_s, int prior_n, int total_items) {
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(kc);
  const uint16_t* v16 = static_cast<const uint16_t*>(vc);
#define MI_LAUNCH_G(GG)                                                                        \
  split_kv_partial_kernel<DT, GG, DTO, kVar, kPR><<<blocks, kThreads, 0, st>>>(                \
      q16, k16, v16, pt, pt_stride, ctx, Hkv, num_phys, num_splits, scale, o_part, lse_part, \
      counters, o, lse, split_indptr, B, prior_o, prior_s, prior_n, total_items)
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
hipError_t launch_dtype(int out_dtype, int G, unsigned blocks, hipStream_t st, const void* q,
                        const void* kc, const void* vc, const int32_t* pt, int pt_stride,
                        const int32_t* ctx, int Hkv, int64_t num_phys, int num_splits, float scale,
                        float* o_part, float* lse_part, int32_t* counters, void* o, float* lse,
                        const int32_t* split_indptr, int B, int total_items,
                        const float* prior_o = nullptr, const float* prior_s = nullptr,
                        int prior_n = 0) {
  // Prior states in registers: one split, at most 16 of them, one head per wave.
  constexpr int kPR = 16;
  if constexpr (!kVar) {
    if (prior_n > 0 && prior_n <= kPR && num_splits == 1 && G <= 4 && out_dtype >= 0) {
      switch (out_dtype) {
        case MI_F16:
          return launch_group<DT, MI_F16, false, kPR>(G, blocks, st, q, kc, vc, pt, pt_stride, ctx, Hkv, num_phys, num_splits, scale, o_part, lse_part, counters, o, lse, split_indptr, B, prior_o, prior_s, prior_n, total_items);
        case MI_BF16:
          return launch_group<DT, MI_BF16, false, kPR>(G, blocks, st, q, kc, vc, pt, pt_stride, ctx, Hkv, num_phys, num_splits, scale, o_part, lse_part, counters, o, lse, split_indptr, B, prior_o, prior_s, prior_n, total_items);
        default:
          return launch_group<DT, MI_F32, false, kPR>(G, blocks, st, q, kc, vc, pt, pt_stride, ctx, Hkv, num_phys, num_splits, scale, o_part, lse_part, counters, o, lse, split_indptr, B, prior_o, prior_s, prior_n, total_items);
      }
    }
  }
  switch (out_dtype) {
    case MI_F16:
      return launch_group<DT, MI_F16, kVar>(G, blocks, st, q, kc, vc, pt, pt_stride, ctx, Hkv, num_phys, num_splits, scale, o_part, lse_part, counters, o, lse, split_indptr, B, prior_o, prior_s, prior_n, total_items);
    case MI_BF16:
      return launch_group<DT, MI_BF16, kVar>(G, blocks, st, q, kc, vc, pt, pt_stride, ctx, Hkv, num_phys, num_splits, scale, o_part, lse_part, counters, o, lse, split_indptr, B, prior_o, prior_s, prior_n, total_items);
    case MI_F32:
      return launch_group<DT, MI_F32, kVar>(G, blocks, st, q, kc, vc, pt, pt_stride, ctx, Hkv, num_phys, num_splits, scale, o_part, lse_part, counters, o, lse, split_indptr, B, prior_o, prior_s, prior_n, total_items);
    default:
      return launch_group<DT, -1, kVar>(G, blocks, st, q, kc, vc, pt, pt_stride, ctx, Hkv, num_phys, num_splits, scale, o_part, lse_part, nullptr, nullptr, nullptr, split_indptr, B, nullptr, nullptr, 0, total_items);
  }
}

// Workgroups for `items` work items of each of Hkv kv heads.
int64_t decode_blocks(int64_t items, int Hkv) { return items * Hkv; }

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
  const int64_t items = static_cast<int64_t>(B) * num_splits;
  const int64_t nblocks = decode_blocks(items, Hkv);
  if (!grid_fits(nblocks, kThreads)) return hipErrorInvalidConfiguration;
  const unsigned blocks = static_cast<unsigned>(nblocks);
  const float scale = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  // o is written by this kernel when fused (counters given) or when there is a
  // single split (no combine needed); otherwise pass 1 only.
  const int dto = (counters != nullptr || (o != nullptr && num_splits == 1)) ? out_dtype : -1;
  if (kv_dtype == MI_F16)
    return launch_dtype<MI_F16, false>(dto, G, blocks, st, q, kc, vc, page_table, pt_stride,
                                       ctx_lens, Hkv, num_phys_pages, num_splits, scale, o_part,
                                       lse_part, counters, o, lse, nullptr, B,
                                       static_cast<int>(items), prior_o, prior_s, prior_n);
  return launch_dtype<MI_BF16, false>(dto, G, blocks, st, q, kc, vc, page_table, pt_stride,
                                      ctx_lens, Hkv, num_phys_pages, num_splits, scale, o_part,
                                      lse_part, counters, o, lse, nullptr, B,
                                      static_cast<int>(items), prior_o, prior_s, prior_n);
}

hipError_t launch_split_kv_partial_varlen(const void* q, const void* kc, const void* vc,
                                          const int32_t* page_table, int pt_stride,
                                          const int32_t* ctx_lens, int B, int Hq, int Hkv,
                                          int64_t num_phys_pages, const int32_t* split_indptr,
                                          int total_splits, float sm_scale, int kv_dtype,
                                          float* o_part, float* lse_part, hipStream_t st,
                                          int32_t* counters, void* o, float* lse, int out_dtype) {
  const int G = Hq / Hkv;
  const int64_t nblocks = decode_blocks(total_splits, Hkv);
  if (!grid_fits(nblocks, kThreads)) return hipErrorInvalidConfiguration;
  const unsigned blocks = static_cast<unsigned>(nblocks);
  const float scale = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  const int dto = counters != nullptr ? out_dtype : -1;
  if (kv_dtype == MI_F16)
    return launch_dtype<MI_F16, true>(dto, G, blocks, st, q, kc, vc, page_table, pt_stride,
                                      ctx_lens, Hkv, num_phys_pages, 0, scale, o_part, lse_part,
                                      counters, o, lse, split_indptr, B, total_splits);
  return launch_dtype<MI_BF16, true>(dto, G, blocks, st, q, kc, vc, page_table, pt_stride,
                                     ctx_lens, Hkv, num_phys_pages, 0, scale, o_part, lse_part,
                                     counters, o, lse, split_indptr, B, total_splits);
}

}  // namespace mi
