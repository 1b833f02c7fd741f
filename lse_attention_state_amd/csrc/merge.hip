// Merge kernels for gfx950: two states per row, and N states per (pos, h).
//
// "F2 hints: merge_state, base-2 LSE merge", sections 3-5: for states with
// base-2 LSEs s_i, m = max s_i, w_i = 2^(s_i - m), v = sum w_i v_i / sum w_i,
// s = m + log2(sum w_i). Both kernels are HBM-bound streams: each lane owns one
// 8-element (16-byte for 16-bit types) chunk of a row, so a row of D = 128 is
// read by 16 consecutive lanes with fully coalesced 16-byte loads (fp32 rows:
// a lane's 8 elements are two 4-element pieces, one in each half of the row,
// so every load instruction of a lane group covers one contiguous run). Every
// load of a row or batch is issued before the first is used (scheduling
// barriers keep the compiler from sinking loads toward their uses, which had
// left one or two in flight). Inputs are loaded with the non-temporal
// (streaming) hint. Output stores: non-temporal, except where fp32 states are
// merged (the split-KV combines and both levels of the two-level merge) into an
// output of at most 64 MiB, small or read back at once by the next level;
// there ordinary write-back stores measured faster on MI355X (S=64 N=1024
// two-level merge 13.4 -> 12.5 us, S*H=1024 N=16 5.4 -> 4.2 us). For large streams
// write-back stores only looked faster while one output buffer was rewritten
// call after call (the Infinity Cache absorbed the rewrites); with the output
// rotated over four buffers they were slower (N-state merge fp16 S=65536 N=4
// H=8: 110.8 -> 114.8 us), and in the two-state merge slower in every mode.
//
// Empty-state handling: incoming s are sanitised (NaN, +inf -> -inf); weights
// use the max-based guard so that -inf - (-inf) gives weight 0; a state of
// weight 0 is skipped by select (its v may hold anything); the normaliser uses
// 1/Z or 0 when Z = 0, so an all-empty row writes v = 0, s = -inf.
//
// The two-state kernel has two more modes: a per-position mask (positions
// whose mask byte is 0 are left untouched: merge_state_in_place, section 7),
// and the attention sink, a second state (0, sink * log2 e) per head
// ("FlashAttention's empty-row LSE", table of section 0, FlashMLA branch of section 2.1).
// The segmented kernel merges index sets of any size, one wave or more per
// (position, head): variable-length segments given by an index pointer array,
// or N states per position when N is too large for the N-state kernel's
// one-pass layout (section 7's "many index sets" variant).
#include "common.h"
#include "launch.h"
#include <type_traits>

namespace mi {
namespace {

constexpr int kBlock = 256;

__host__ __device__ constexpr int log2_int(int x) { return x <= 1 ? 0 : 1 + log2_int(x >> 1); }

int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// fp32 rows in two halves: lane c holds elements [4c, 4c + 4) and
// [D/2 + 4c, D/2 + 4c + 4), so each load instruction of a lane group reads
// one contiguous run of 16 L bytes (D = 8 L).
// Raw words as for load8_raw<MI_F32>; unpack8_raw<MI_F32> gives the lane's
// elements in the order [4c, 4c + 4) then [D/2 + 4c, D/2 + 4c + 4).
__device__ __forceinline__ Raw8 load8_halves_raw(const float* row, int c, int half) {
  Raw8 r;
  r.a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row + 4 * c));
  r.b = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row + half + 4 * c));
  return r;
}

// The output of a row merged from fp32 halves, in the same lane layout:
// write-back stores when `wb` (a small output, see the file header), else
// non-temporal ones.
template <int DT>
__device__ __forceinline__ void store8_halves(void* base, int64_t rowoff, int c, int half,
                                              const float (&x)[8], bool wb) {
  if constexpr (DT == MI_F32) {
    float* row = static_cast<float*>(base) + rowoff;
    const float4_t a{x[0], x[1], x[2], x[3]}, b{x[4], x[5], x[6], x[7]};
    if (wb) {
      *reinterpret_cast<float4_t*>(row + 4 * c) = a;
      *reinterpret_cast<float4_t*>(row + half + 4 * c) = b;
    } else {
      __builtin_nontemporal_store(a, reinterpret_cast<float4_t*>(row + 4 * c));
      __builtin_nontemporal_store(b, reinterpret_cast<float4_t*>(row + half + 4 * c));
    }
  } else {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    uint16_t* row = static_cast<uint16_t*>(base) + rowoff;
    const u32x2_t lo = (DT == MI_F16) ? u32x2_t{pack_f16(x[0], x[1]), pack_f16(x[2], x[3])}
                                      : u32x2_t{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
    const u32x2_t hi = (DT == MI_F16) ? u32x2_t{pack_f16(x[4], x[5]), pack_f16(x[6], x[7])}
                                      : u32x2_t{pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
    if (wb) {
      *reinterpret_cast<u32x2_t*>(row + 4 * c) = lo;
      *reinterpret_cast<u32x2_t*>(row + half + 4 * c) = hi;
    } else {
      __builtin_nontemporal_store(lo, reinterpret_cast<u32x2_t*>(row + 4 * c));
      __builtin_nontemporal_store(hi, reinterpret_cast<u32x2_t*>(row + half + 4 * c));
    }
  }
}

// Outputs up to this size take write-back stores in the fp32-state merges.
constexpr int64_t kWriteBackMaxBytes = int64_t(64) << 20;

// Two states. Lanes per row L = 2^lanes_shift >= D/8; a block covers 256/L rows.
// MODE: kPlain; kMasked (mask [rows / H] bytes, 0 = keep state a untouched);
// kSink (state b is (0, sink[row % H] * log2 e); vb and sb are unused).
enum { kPlain = 0, kMasked = 1, kSink = 2 };
constexpr float kLog2e = 1.4426950408889634f;

template <int DTI, int DTO, int MODE>
__global__ __launch_bounds__(kBlock) void merge_state_kernel(
    const void* va, const float* sa, const void* vb, const float* sb, void* vo, float* so,
    int64_t rows, int D, int lanes_shift, const uint8_t* mask, const float* sink, int H) {
  const int lane_in_row = threadIdx.x & ((1 << lanes_shift) - 1);
  const int64_t row =
      static_cast<int64_t>(blockIdx.x) * (kBlock >> lanes_shift) + (threadIdx.x >> lanes_shift);
  if (row >= rows) return;
  if constexpr (MODE == kMasked) {
    if (mask[row / H] == 0) return;
  }
  // All loads of the row are issued before any is used: the state loads do not
  // wait for the LSE loads. Lanes past D read the row's first chunk (in
  // bounds) and store nothing.
  const int d0 = lane_in_row * 8;
  const int64_t off = row * D + (d0 < D ? d0 : 0);
  const Raw8 ra = load8_raw<DTI>(va, off);
  Raw8 rb;
  if constexpr (MODE != kSink) rb = load8_raw<DTI>(vb, off);
  const float sa_raw = sa[row];
  float sb_raw;
  if constexpr (MODE == kSink)
    sb_raw = sink[row % H] * kLog2e;
  else
    sb_raw = sb[row];
  __builtin_amdgcn_sched_barrier(0);
  float xa[8], xb[8];
  unpack8_raw<DTI>(ra, xa);
  if constexpr (MODE != kSink) unpack8_raw<DTI>(rb, xb);
  const float a = sanitize_lse(sa_raw);
  const float b = sanitize_lse(sb_raw);
  const float m = __builtin_fmaxf(a, b);
  const float wa = guarded_exp2(a - m);
  const float wb = guarded_exp2(b - m);
  const float z = wa + wb;
  if (d0 < D) {
    float y[8];
    const float inv = guarded_inv(z);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // Two rounded products and one add: the same bits for (a, b) and (b, a).
      const float ta = (wa > 0.0f) ? wa * xa[j] : 0.0f;
      const float tb = (MODE != kSink && wb > 0.0f) ? wb * xb[j] : 0.0f;
      y[j] = (ta + tb) * inv;
    }
    store8<DTO, true>(vo, off, y);
  }
  // In-place use may alias so with sa/sb: every lane of the row has read them
  // above, and a row's lanes (D <= 512, so at most 64) sit in one wave.
  if (so != nullptr && lane_in_row == 0) so[row] = m + hw_log2(z);
}


// N states. Each row (pos, h) is served by G = 2^groups_shift groups of L lanes;
// group g handles states n = g, g+G, ...; groups are merged through LDS.
constexpr int kLdsFloats = 2048 + 512;  // rows_per_block * G * (8L + 2) <= 2048 + 512/L

template <int DTI, int DTO, int kChunk, bool kHalves = false>
__global__ __launch_bounds__(kBlock) void merge_states_kernel(
    const void* __restrict__ v, const float* __restrict__ s, void* __restrict__ vo,
    float* __restrict__ so, int64_t rows, int N, int H, int D, int lanes_shift,
    int groups_shift, int wb) {
  __shared__ float lds[kLdsFloats];
  const int L = 1 << lanes_shift;
  const int G = 1 << groups_shift;
  const int lane_in_row = threadIdx.x & (L - 1);
  const int g = (threadIdx.x >> lanes_shift) & (G - 1);
  const int row_in_block = threadIdx.x >> (lanes_shift + groups_shift);
  const int rows_per_block = kBlock >> (lanes_shift + groups_shift);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * rows_per_block + row_in_block;
  const bool row_ok = row < rows;
  const int d0 = lane_in_row * 8;
  const bool lane_ok = d0 < D;
  const int64_t pos = row_ok ? row / H : 0;
  const int h = row_ok ? static_cast<int>(row - pos * H) : 0;

  // The group's states are taken kChunk at a time: all of a chunk's s and v
  // loads are issued before any is used (so they are in flight together), then
  // the chunk is folded into the running state (m, z, acc) with the merge rule.
  float m = -kInf;
  float z = 0.0f;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  if (row_ok) {
    for (int n0 = g; n0 < N; n0 += kChunk * G) {
      float sv[kChunk];
      Raw8 xr[kChunk];
      // Loads are unconditional (indices clamped to valid ones) and results
      // are selected afterwards: a load under a lane mask followed by a
      // zero-fill of the same registers would force a wait after every load.
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const int n = n0 + u * G;
        const int64_t idx = (pos * N + (n < N ? n : 0)) * H + h;
        sv[u] = s[idx];
        if constexpr (kHalves)
          xr[u] = load8_halves_raw(static_cast<const float*>(v) + idx * D, lane_in_row, D / 2);
        else
          xr[u] = load8_raw<DTI>(v, idx * D + (lane_ok ? d0 : 0));
      }
      __builtin_amdgcn_sched_barrier(0);
      float x[kChunk][8];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) unpack8_raw<DTI>(xr[u], x[u]);
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const bool in = n0 + u * G < N;
        sv[u] = in ? sanitize_lse(sv[u]) : -kInf;
        // A state past N gets weight 0 and the guarded FMA below skips it, so
        // its clamped load (possibly NaN) never reaches acc; lanes past D are
        // never stored. The zero-fill is therefore redundant: without it,
        // chunks of 8 states run 10% faster (S=512 N=64 H=8 fp16: 16.2 ->
        // 14.5 us); with 4 or fewer it measured 1-2% faster kept, so it stays.
        if constexpr (kChunk < 8) {
#pragma unroll
          for (int j = 0; j < 8; ++j) x[u][j] = (in && lane_ok) ? x[u][j] : 0.0f;
        }
      }
      float cm = m;
#pragma unroll
      for (int u = 0; u < kChunk; ++u) cm = __builtin_fmaxf(cm, sv[u]);
      const float keep = guarded_exp2(m - cm);
      z *= keep;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= keep;
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const float w = guarded_exp2(sv[u] - cm);
        z += w;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = (w > 0.0f) ? __builtin_fmaf(w, x[u][j], acc[j]) : acc[j];
      }
      m = cm;
    }
  }

  if (G > 1) {
    const int stride = 8 * L + 2;
    float* mine = lds + (row_in_block * G + g) * stride;
#pragma unroll
    for (int j = 0; j < 8; ++j) mine[d0 + j] = acc[j];
    if (lane_in_row == 0) {
      mine[8 * L] = m;
      mine[8 * L + 1] = z;
    }
    __syncthreads();
    if (g != 0) return;
    const float* grp = lds + row_in_block * G * stride;
    float M = -kInf;
    for (int k = 0; k < G; ++k) M = __builtin_fmaxf(M, grp[k * stride + 8 * L]);
    z = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
    for (int k = 0; k < G; ++k) {
      const float* gk = grp + k * stride;
      const float w = guarded_exp2(gk[8 * L] - M);
      z = __builtin_fmaf(w, gk[8 * L + 1], z);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = (w > 0.0f) ? __builtin_fmaf(w, gk[d0 + j], acc[j]) : acc[j];
    }
    m = M;
  }
  if (!row_ok) return;
  if (lane_ok) {
    const float inv = guarded_inv(z);
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = acc[j] * inv;
    if constexpr (kHalves)
      store8_halves<DTO>(vo, row * D, lane_in_row, D / 2, y, wb != 0);
    else
      store8<DTO, true>(vo, row * D + d0, y);
  }
  if (so != nullptr && lane_in_row == 0) so[row] = m + hw_log2(z);
}

template <int DTI, int MODE>
hipError_t merge_state_out(int dt_out, const void* va, const float* sa, const void* vb,
                           const float* sb, void* vo, float* so, int64_t rows, int D,
                           int lanes_shift, const uint8_t* mask, const float* sink, int H,
                           dim3 grid, hipStream_t st) {
  switch (dt_out) {
    case MI_F16:
      merge_state_kernel<DTI, MI_F16, MODE><<<grid, kBlock, 0, st>>>(va, sa, vb, sb, vo, so, rows, D, lanes_shift, mask, sink, H);
      break;
    case MI_BF16:
      merge_state_kernel<DTI, MI_BF16, MODE><<<grid, kBlock, 0, st>>>(va, sa, vb, sb, vo, so, rows, D, lanes_shift, mask, sink, H);
      break;
    default:
      merge_state_kernel<DTI, MI_F32, MODE><<<grid, kBlock, 0, st>>>(va, sa, vb, sb, vo, so, rows, D, lanes_shift, mask, sink, H);
      break;
  }
  return hipGetLastError();
}

template <int MODE>
hipError_t merge_state_mode(const void* va, const float* sa, const void* vb, const float* sb,
                            void* vo, float* so, int64_t rows, int D, int dt_in, int dt_out,
                            const uint8_t* mask, const float* sink, int H, hipStream_t st) {
  const int lanes_shift = log2_int(next_pow2(D / 8));
  const int64_t rows_per_block = kBlock >> lanes_shift;
  const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  if (!grid_fits(blocks, kBlock)) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  switch (dt_in) {
    case MI_F16: return merge_state_out<MI_F16, MODE>(dt_out, va, sa, vb, sb, vo, so, rows, D, lanes_shift, mask, sink, H, grid, st);
    case MI_BF16: return merge_state_out<MI_BF16, MODE>(dt_out, va, sa, vb, sb, vo, so, rows, D, lanes_shift, mask, sink, H, grid, st);
    default: return merge_state_out<MI_F32, MODE>(dt_out, va, sa, vb, sb, vo, so, rows, D, lanes_shift, mask, sink, H, grid, st);
  }
}


// Segmented merge: row (pos, h) merges the states start..end-1 of v [total, H, D],
// s [total, H], where [start, end) = [indptr[pos], indptr[pos+1]) clamped to
// [0, total], or [pos*N, (pos+1)*N) when indptr is null (the N-state layout
// [S, N, H, D] is the same memory). A row is served by a team of
// T = 2^team_shift lanes: G = T / L lane groups of L = 2^lanes_shift lanes,
// each group covering one state's D and taking states g, g + G, ... Short
// segments get small teams (several rows per wave, like the N-state kernel);
// long ones get teams of up to 16 waves, so even a few rows with thousands of
// states keep the device's memory pipeline full. A lane keeps K states' loads
// in flight and folds them into its running (m, z, acc); the groups then merge
// across lanes, and the waves of a team through LDS.
// Block size: 256 threads while a team fits in it (more blocks per compute
// unit), 1024 for teams of more than four waves.
constexpr int kSegMaxD = 512;

// parts > 1 (no indptr): each position's N states are cut into `parts`
// consecutive slices of ceil(N / parts), and row (pos * parts + part) * H + h
// merges one slice -- the first level of a two-level merge.
template <int DTI, int DTO, int K, int kSegThreads, bool kHalves = false>
__global__ __launch_bounds__(kSegThreads) void merge_segments_kernel(
    const void* __restrict__ v, const float* __restrict__ s, const int32_t* __restrict__ indptr,
    int64_t total, int N, void* __restrict__ vo, float* __restrict__ so, int64_t rows, int H,
    int D, int lanes_shift, int team_shift, int parts, int wb) {
  __shared__ float lds_acc[kSegThreads / 64][kSegMaxD];
  __shared__ float lds_mz[kSegThreads / 64][2];
  const int L = 1 << lanes_shift;
  const int T = 1 << team_shift;
  const int G = T >> lanes_shift;
  const int t = threadIdx.x & (T - 1);
  const int c = t & (L - 1);
  const int g = t >> lanes_shift;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kSegThreads >> team_shift) +
                      (threadIdx.x >> team_shift);
  const bool row_ok = row < rows;
  const int d0 = c * 8;
  const bool lane_ok = d0 < D;
  const int64_t ph = row_ok ? row / H : 0;   // position (and slice)
  const int h = row_ok ? static_cast<int>(row - ph * H) : 0;
  int64_t start = 0, end = 0;
  if (row_ok) {
    if (indptr != nullptr) {
      start = indptr[ph];
      end = indptr[ph + 1];
      start = start < 0 ? 0 : (start > total ? total : start);
      end = end < start ? start : (end > total ? total : end);
    } else if (parts == 1) {
      start = ph * N;
      end = start + N;
    } else {
      const int64_t pos = ph / parts;
      const int64_t per = (N + parts - 1) / parts;
      const int64_t last = pos * N + N;
      start = pos * N + (ph - pos * parts) * per;
      start = start < last ? start : last;
      end = start + per < last ? start + per : last;
    }
  }
  const int64_t n = end - start;

  float m = -kInf, z = 0.0f, acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
  // States are folded in batches of KK per lane (KK <= K), all of a batch's
  // loads in flight together. The batch size is the smallest power of two
  // that covers what the wave's lanes still have, so short sets issue no
  // loads for states they do not have. Lanes whose set is done (or empty)
  // take part with every state masked; their loads use an index that exists
  // (the set's first state, or state 0 of the array for an empty set: some
  // lane of the wave still has states, so the arrays are not empty).
  auto fold = [&](auto kk, int64_t k0) {
    constexpr int KK = decltype(kk)::value;
    float sv[KK];
    Raw8 xr[KK];
#pragma unroll
    for (int u = 0; u < KK; ++u) {
      const int64_t k = k0 + static_cast<int64_t>(u) * G;
      const int64_t idx = (k < n ? start + k : (n > 0 ? start : 0)) * H + h;
      sv[u] = s[idx];
      if constexpr (kHalves)
        xr[u] = load8_halves_raw(static_cast<const float*>(v) + idx * D, c, D / 2);
      else
        xr[u] = load8_raw<DTI>(v, idx * D + (lane_ok ? d0 : 0));
    }
    __builtin_amdgcn_sched_barrier(0);
    float x[KK][8];
#pragma unroll
    for (int u = 0; u < KK; ++u) unpack8_raw<DTI>(xr[u], x[u]);
    float cm = m;
#pragma unroll
    for (int u = 0; u < KK; ++u) {
      sv[u] = (k0 + static_cast<int64_t>(u) * G < n) ? sanitize_lse(sv[u]) : -kInf;
      cm = __builtin_fmaxf(cm, sv[u]);
    }
    const float keep = guarded_exp2(m - cm);
    z *= keep;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= keep;
#pragma unroll
    for (int u = 0; u < KK; ++u) {
      const float w = guarded_exp2(sv[u] - cm);
      z += w;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = (w > 0.0f && lane_ok) ? __builtin_fmaf(w, x[u][j], acc[j]) : acc[j];
    }
    m = cm;
  };
  for (int64_t k0 = g;;) {
    const int64_t rem = n - k0;
    if (K >= 8 && __builtin_amdgcn_ballot_w64(rem > 4 * static_cast<int64_t>(G)) != 0) {
      fold(std::integral_constant<int, (K >= 8 ? 8 : 1)>{}, k0);
      k0 += 8 * static_cast<int64_t>(G);
    } else if (K >= 4 && __builtin_amdgcn_ballot_w64(rem > 2 * static_cast<int64_t>(G)) != 0) {
      fold(std::integral_constant<int, (K >= 4 ? 4 : 1)>{}, k0);
      k0 += 4 * static_cast<int64_t>(G);
    } else if (K >= 2 && __builtin_amdgcn_ballot_w64(rem > static_cast<int64_t>(G)) != 0) {
      fold(std::integral_constant<int, (K >= 2 ? 2 : 1)>{}, k0);
      k0 += 2 * static_cast<int64_t>(G);
    } else if (__builtin_amdgcn_ballot_w64(rem > 0) != 0) {
      fold(std::integral_constant<int, 1>{}, k0);
      k0 += static_cast<int64_t>(G);
    } else {
      break;
    }
  }
  // Merge the lane groups inside each wave (lanes c, c + L, c + 2L, ... of the team).
  const int in_wave = T < 64 ? T : 64;
  for (int sh = L; sh < in_wave; sh <<= 1) {
    const float mo = shfl_xor(m, sh);
    const float zo = shfl_xor(z, sh);
    const float M = __builtin_fmaxf(m, mo);
    const float ws = guarded_exp2(m - M);
    const float wo = guarded_exp2(mo - M);
    z = z * ws + zo * wo;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = acc[j] * ws + shfl_xor(acc[j], sh) * wo;
    m = M;
  }
  if (T > 64) {
    // Teams of several waves: each wave's lanes of group 0 (t < L within the
    // wave) hold the wave's merge; the team's first wave folds them.
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    if (lane < L && lane_ok) {
#pragma unroll
      for (int j = 0; j < 8; ++j) lds_acc[wave][d0 + j] = acc[j];
    }
    if (lane == 0) {
      lds_mz[wave][0] = m;
      lds_mz[wave][1] = z;
    }
    __syncthreads();
    const int W = T >> 6;
    if ((wave & (W - 1)) != 0) return;
    float M = -kInf;
    for (int k = 0; k < W; ++k) M = __builtin_fmaxf(M, lds_mz[wave + k][0]);
    z = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
    for (int k = 0; k < W; ++k) {
      const float w = guarded_exp2(lds_mz[wave + k][0] - M);
      z = __builtin_fmaf(w, lds_mz[wave + k][1], z);
      if (w > 0.0f && lane_ok) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_fmaf(w, lds_acc[wave + k][d0 + j], acc[j]);
      }
    }
    m = M;
  }
  if (!row_ok || g != 0) return;
  if (lane_ok) {
    const float inv = guarded_inv(z);
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = acc[j] * inv;
    if constexpr (kHalves)
      store8_halves<DTO>(vo, row * D, c, D / 2, y, wb != 0);
    else
      store8<DTO, true>(vo, row * D + d0, y);
  }
  if (so != nullptr && c == 0) so[row] = m + hw_log2(z);
}

template <int DTI, int DTO, int kThr, bool kH = false>
hipError_t merge_segments_kt(int K, dim3 grid, hipStream_t st, const void* v, const float* s,
                             const int32_t* indptr, int64_t total, int N, void* vo, float* so,
                             int64_t rows, int H, int D, int lanes_shift, int team_shift,
                             int parts, int wb) {
  switch (K) {
    case 1:
      merge_segments_kernel<DTI, DTO, 1, kThr, kH><<<grid, kThr, 0, st>>>(v, s, indptr, total, N, vo, so, rows, H, D, lanes_shift, team_shift, parts, wb);
      break;
    case 2:
      merge_segments_kernel<DTI, DTO, 2, kThr, kH><<<grid, kThr, 0, st>>>(v, s, indptr, total, N, vo, so, rows, H, D, lanes_shift, team_shift, parts, wb);
      break;
    case 4:
      merge_segments_kernel<DTI, DTO, 4, kThr, kH><<<grid, kThr, 0, st>>>(v, s, indptr, total, N, vo, so, rows, H, D, lanes_shift, team_shift, parts, wb);
      break;
    default:
      merge_segments_kernel<DTI, DTO, 8, kThr, kH><<<grid, kThr, 0, st>>>(v, s, indptr, total, N, vo, so, rows, H, D, lanes_shift, team_shift, parts, wb);
      break;
  }
  return hipGetLastError();
}

// The grid is given in teams; the block size follows from the team size.
template <int DTI, int DTO>
hipError_t merge_segments_k(int K, int64_t rows, hipStream_t st, const void* v, const float* s,
                            const int32_t* indptr, int64_t total, int N, void* vo, float* so,
                            int H, int D, int lanes_shift, int team_shift, int parts) {
  const int threads = team_shift > 8 ? 1024 : 256;
  const int64_t rows_per_block = threads >> team_shift;
  const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  if (!grid_fits(blocks, threads)) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  const int wb = rows * D * (DTO == MI_F32 ? 4 : 2) <= kWriteBackMaxBytes;
  if constexpr (DTI == MI_F32) {
    if (D == (8 << lanes_shift)) {
      if (threads == 1024)
        return merge_segments_kt<DTI, DTO, 1024, true>(K, grid, st, v, s, indptr, total, N, vo, so, rows, H, D, lanes_shift, team_shift, parts, wb);
      return merge_segments_kt<DTI, DTO, 256, true>(K, grid, st, v, s, indptr, total, N, vo, so, rows, H, D, lanes_shift, team_shift, parts, wb);
    }
  }
  if (threads == 1024)
    return merge_segments_kt<DTI, DTO, 1024>(K, grid, st, v, s, indptr, total, N, vo, so, rows, H, D, lanes_shift, team_shift, parts, wb);
  return merge_segments_kt<DTI, DTO, 256>(K, grid, st, v, s, indptr, total, N, vo, so, rows, H, D, lanes_shift, team_shift, parts, wb);
}

template <int DTI>
hipError_t merge_segments_out(int dt_out, int K, int64_t rows, hipStream_t st, const void* v,
                              const float* s, const int32_t* indptr, int64_t total, int N,
                              void* vo, float* so, int H, int D, int lanes_shift, int team_shift,
                              int parts) {
  switch (dt_out) {
    case MI_F16:
      return merge_segments_k<DTI, MI_F16>(K, rows, st, v, s, indptr, total, N, vo, so, H, D, lanes_shift, team_shift, parts);
    case MI_BF16:
      return merge_segments_k<DTI, MI_BF16>(K, rows, st, v, s, indptr, total, N, vo, so, H, D, lanes_shift, team_shift, parts);
    default:
      return merge_segments_k<DTI, MI_F32>(K, rows, st, v, s, indptr, total, N, vo, so, H, D, lanes_shift, team_shift, parts);
  }
}

template <int DTI, int DTO, bool kH>
hipError_t merge_states_chunk(int chunk, const void* v, const float* s, void* vo, float* so,
                              int64_t rows, int N, int H, int D, int lanes_shift,
                              int groups_shift, dim3 grid, hipStream_t st) {
  const int wb = rows * D * (DTO == MI_F32 ? 4 : 2) <= kWriteBackMaxBytes;
  switch (chunk) {
    case 1:
      merge_states_kernel<DTI, DTO, 1, kH><<<grid, kBlock, 0, st>>>(v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift, wb);
      break;
    case 2:
      merge_states_kernel<DTI, DTO, 2, kH><<<grid, kBlock, 0, st>>>(v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift, wb);
      break;
    case 4:
      merge_states_kernel<DTI, DTO, 4, kH><<<grid, kBlock, 0, st>>>(v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift, wb);
      break;
    default:
      merge_states_kernel<DTI, DTO, 8, kH><<<grid, kBlock, 0, st>>>(v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift, wb);
      break;
  }
  return hipGetLastError();
}

template <int DTI, bool kH = false>
hipError_t merge_states_out(int dt_out, int chunk, const void* v, const float* s, void* vo,
                            float* so, int64_t rows, int N, int H, int D, int lanes_shift,
                            int groups_shift, dim3 grid, hipStream_t st) {
  switch (dt_out) {
    case MI_F16:
      return merge_states_chunk<DTI, MI_F16, kH>(chunk, v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift, grid, st);
    case MI_BF16:
      return merge_states_chunk<DTI, MI_BF16, kH>(chunk, v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift, grid, st);
    default:
      return merge_states_chunk<DTI, MI_F32, kH>(chunk, v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift, grid, st);
  }
}

}  // namespace

hipError_t launch_merge_state(const void* va, const float* sa, const void* vb, const float* sb,
                              void* vo, float* so, int64_t rows, int D, int dt_in, int dt_out,
                              hipStream_t st) {
  return merge_state_mode<kPlain>(va, sa, vb, sb, vo, so, rows, D, dt_in, dt_out, nullptr,
                                  nullptr, 1, st);
}

hipError_t launch_merge_state_masked(void* v, float* s, const void* v_other,
                                     const float* s_other, const uint8_t* mask, int64_t rows,
                                     int H, int D, int dt, hipStream_t st) {
  if (mask == nullptr)
    return merge_state_mode<kPlain>(v, s, v_other, s_other, v, s, rows, D, dt, dt, nullptr,
                                    nullptr, H, st);
  return merge_state_mode<kMasked>(v, s, v_other, s_other, v, s, rows, D, dt, dt, mask, nullptr,
                                   H, st);
}

hipError_t launch_merge_sink(const void* v, const float* s, const float* sink, void* vo,
                             float* so, int64_t rows, int H, int D, int dt_in, int dt_out,
                             hipStream_t st) {
  return merge_state_mode<kSink>(v, s, nullptr, nullptr, vo, so, rows, D, dt_in, dt_out,
                                 nullptr, sink, H, st);
}

hipError_t launch_merge_segments(const void* v, const float* s, const int32_t* indptr,
                                 int64_t total, int N, void* vo, float* so, int64_t S, int H,
                                 int D, int dt_in, int dt_out, hipStream_t st, int parts) {
  const int64_t rows = S * parts * H;
  const int L = next_pow2(D / 8);
  const int lanes_shift = log2_int(L);
  // Team size from the average set size: up to 8 states per lane per batch,
  // in teams of at most 256 lanes while rows are plentiful (several
  // workgroups per compute unit keep its memory pipeline busy while one of
  // them merges: measured on MI355X, S*H = 2048 slices of 512 fp32 states in
  // 87 us against 107 us with teams of 1024); more lane groups (up to 16
  // waves per row, while each group keeps at least 4 states) when there are
  // too few rows to give the device about 16 waves per compute unit. (At one
  // state per group the cross-group merge outweighed the extra loads in
  // flight: the split combine of 32 rows x 64 fp32 partials took 5.2 us per
  // call against 4.0 us with 4 states per group.)
  const int64_t avg = indptr != nullptr ? (S > 0 ? (total + S - 1) / S : 0)
                                        : (static_cast<int64_t>(N) + parts - 1) / parts;
  constexpr int64_t kTargetLanes = 4096 * 64;
  constexpr int kMinStatesPerGroup = 4;
  const int max_groups = 1024 / L;
  const int batch_groups = 256 / L < max_groups ? 256 / L : max_groups;
  int G = 1;
  while (G < batch_groups && static_cast<int64_t>(G) * 8 < avg) G *= 2;
  while (G < max_groups && static_cast<int64_t>(2 * G) * kMinStatesPerGroup <= avg &&
         rows * L * G < kTargetLanes)
    G *= 2;
  const int team_shift = log2_int(L * G);
  const int64_t per_lane = (avg + G - 1) / G;
  const int K = per_lane >= 8 ? 8 : next_pow2(static_cast<int>(per_lane > 0 ? per_lane : 1));
  switch (dt_in) {
    case MI_F16: return merge_segments_out<MI_F16>(dt_out, K, rows, st, v, s, indptr, total, N, vo, so, H, D, lanes_shift, team_shift, parts);
    case MI_BF16: return merge_segments_out<MI_BF16>(dt_out, K, rows, st, v, s, indptr, total, N, vo, so, H, D, lanes_shift, team_shift, parts);
    default: return merge_segments_out<MI_F32>(dt_out, K, rows, st, v, s, indptr, total, N, vo, so, H, D, lanes_shift, team_shift, parts);
  }
}

int merge_states_parts(int64_t S, int N, int H) {
  // Two levels only when rows alone give the device few workgroups: cut each
  // row's states into slices of at least 64 until there are about 2048 rows.
  // (Measured on MI355X: slices of at least 64 states and about 2048 rows beat
  // 32 or 16 states and 4096 or 8192 rows.)
  const int64_t rows = S * H;
  int parts = 1;
  while (parts < 64 && rows * parts < 2048 && N / (2 * parts) >= 64) parts *= 2;
  return parts;
}

hipError_t launch_merge_states_two_level(const void* v, const float* s, void* vo, float* so,
                                         int64_t S, int N, int H, int D, int dt_in, int dt_out,
                                         float* ws, hipStream_t st) {
  const int parts = merge_states_parts(S, N, H);
  if (parts == 1) return launch_merge_states(v, s, vo, so, S, N, H, D, dt_in, dt_out, st);
  // Level 1: slice states -> fp32 partial states [S, parts, H, D] and [S, parts, H].
  float* wv = ws;
  float* wsl = ws + S * parts * H * D;
  hipError_t e = launch_merge_segments(v, s, nullptr, S * N, N, wv, wsl, S, H, D, dt_in, MI_F32,
                                       st, parts);
  if (e != hipSuccess) return e;
  // Level 2: the N-state merge of the partials ([S, parts, H, D] is that layout).
  return launch_merge_segments(wv, wsl, nullptr, S * parts, parts, vo, so, S, H, D, MI_F32,
                               dt_out, st, 1);
}

hipError_t launch_merge_states(const void* v, const float* s, void* vo, float* so, int64_t S,
                               int N, int H, int D, int dt_in, int dt_out, hipStream_t st) {
  const int64_t rows = S * H;
  // Few rows with many states each (the split-KV combine at small batch): the
  // segmented kernel spreads a row over up to 16 waves (measured on MI355X:
  // S*H = 32, N = 64 fp32 in 8.4 us against 11.6; S*H = 1024, N = 16 in 8.1
  // against 8.8); with many rows the N-state kernel's lighter merge wins.
  if (rows < 2048 && N >= 8)
    return launch_merge_segments(v, s, nullptr, S * N, N, vo, so, S, H, D, dt_in, dt_out, st, 1);
  const int L = next_pow2(D / 8);
  const int lanes_shift = log2_int(L);
  // Split the N states of a row over G lane groups when rows alone would not
  // give the device enough independent loads in flight.
  constexpr int64_t kTargetThreads = 16 * 1024;
  int G = 1;
  while (G < N && G * L < kBlock && rows * L * G < kTargetThreads) G *= 2;
  const int groups_shift = log2_int(G);
  // States per group per chunk: enough to cover a group's share in one pass
  // when it is small, at most 8.
  const int per_group = (N + G - 1) / G;
  const int chunk = per_group >= 8 ? 8 : next_pow2(per_group);
  const int64_t rows_per_block = kBlock >> (lanes_shift + groups_shift);
  const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  if (!grid_fits(blocks, kBlock)) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
  switch (dt_in) {
    case MI_F16: return merge_states_out<MI_F16>(dt_out, chunk, v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift, grid, st);
    case MI_BF16: return merge_states_out<MI_BF16>(dt_out, chunk, v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift, grid, st);
    default:
      // fp32 rows in halves (whole-row runs per load instruction) when D = 8 L.
      if (D == (8 << lanes_shift))
        return merge_states_out<MI_F32, true>(dt_out, chunk, v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift, grid, st);
      return merge_states_out<MI_F32>(dt_out, chunk, v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift, grid, st);
  }
}

}  // namespace mi
