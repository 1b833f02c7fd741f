// Merge kernels for gfx950: two states per row, and N states per (pos, h).
//
// "F2 hints: merge_state, base-2 LSE merge", sections 3-5: for states with
// base-2 LSEs s_i, m = max s_i, w_i = 2^(s_i - m), v = sum w_i v_i / sum w_i,
// s = m + log2(sum w_i). Both kernels are HBM-bound streams: each lane owns one
// 8-element (16-byte for 16-bit types) chunk of a row, so a row of D = 128 is
// read by 16 consecutive lanes with fully coalesced 16-byte loads.
//
// Empty-state handling: incoming s are sanitised (NaN, +inf -> -inf); weights
// use the max-based guard so that -inf - (-inf) gives weight 0; a state of
// weight 0 is skipped by select (its v may hold anything); the normaliser uses
// 1/Z or 0 when Z = 0, so an all-empty row writes v = 0, s = -inf.
#include "common.h"
#include "launch.h"

namespace mi {
namespace {

constexpr int kBlock = 256;

__host__ __device__ constexpr int log2_int(int x) { return x <= 1 ? 0 : 1 + log2_int(x >> 1); }

int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Two states. Lanes per row L = 2^lanes_shift >= D/8; a block covers 256/L rows.
template <int DTI, int DTO>
__global__ __launch_bounds__(kBlock) void merge_state_kernel(
    const void* va, const float* sa, const void* vb, const float* sb, void* vo, float* so,
    int64_t rows, int D, int lanes_shift) {
  const int lane_in_row = threadIdx.x & ((1 << lanes_shift) - 1);
  const int64_t row =
      static_cast<int64_t>(blockIdx.x) * (kBlock >> lanes_shift) + (threadIdx.x >> lanes_shift);
  if (row >= rows) return;
  const float a = sanitize_lse(sa[row]);
  const float b = sanitize_lse(sb[row]);
  const float m = __builtin_fmaxf(a, b);
  const float wa = guarded_exp2(a - m);
  const float wb = guarded_exp2(b - m);
  const float z = wa + wb;
  const int d0 = lane_in_row * 8;
  if (d0 < D) {
    const int64_t off = row * D + d0;
    float xa[8], xb[8], y[8];
    load8<DTI>(va, off, xa);
    load8<DTI>(vb, off, xb);
    const float inv = guarded_inv(z);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // Two rounded products and one add: the same bits for (a, b) and (b, a).
      const float ta = (wa > 0.0f) ? wa * xa[j] : 0.0f;
      const float tb = (wb > 0.0f) ? wb * xb[j] : 0.0f;
      y[j] = (ta + tb) * inv;
    }
    store8<DTO>(vo, off, y);
  }
  // In-place use may alias so with sa/sb: every lane of the row has read them
  // above, and a row's lanes (D <= 512, so at most 64) sit in one wave.
  if (so != nullptr && lane_in_row == 0) so[row] = m + hw_log2(z);
}

// N states. Each row (pos, h) is served by G = 2^groups_shift groups of L lanes;
// group g handles states n = g, g+G, ...; groups are merged through LDS.
constexpr int kLdsFloats = 2048 + 512;  // rows_per_block * G * (8L + 2) <= 2048 + 512/L

template <int DTI, int DTO, int kChunk>
__global__ __launch_bounds__(kBlock) void merge_states_kernel(
    const void* __restrict__ v, const float* __restrict__ s, void* __restrict__ vo,
    float* __restrict__ so, int64_t rows, int N, int H, int D, int lanes_shift,
    int groups_shift) {
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
      float x[kChunk][8];
      // Loads are unconditional (indices clamped to valid ones) and results
      // are selected afterwards: a load under a lane mask followed by a
      // zero-fill of the same registers would force a wait after every load.
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const int n = n0 + u * G;
        const int64_t idx = (pos * N + (n < N ? n : 0)) * H + h;
        sv[u] = s[idx];
        load8<DTI>(v, idx * D + (lane_ok ? d0 : 0), x[u]);
      }
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const bool in = n0 + u * G < N;
        sv[u] = in ? sanitize_lse(sv[u]) : -kInf;
#pragma unroll
        for (int j = 0; j < 8; ++j) x[u][j] = (in && lane_ok) ? x[u][j] : 0.0f;
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
    store8<DTO>(vo, row * D + d0, y);
  }
  if (so != nullptr && lane_in_row == 0) so[row] = m + hw_log2(z);
}

template <int DTI>
hipError_t merge_state_out(int dt_out, const void* va, const float* sa, const void* vb,
                           const float* sb, void* vo, float* so, int64_t rows, int D,
                           int lanes_shift, dim3 grid, hipStream_t st) {
  switch (dt_out) {
    case MI_F16:
      merge_state_kernel<DTI, MI_F16><<<grid, kBlock, 0, st>>>(va, sa, vb, sb, vo, so, rows, D, lanes_shift);
      break;
    case MI_BF16:
      merge_state_kernel<DTI, MI_BF16><<<grid, kBlock, 0, st>>>(va, sa, vb, sb, vo, so, rows, D, lanes_shift);
      break;
    default:
      merge_state_kernel<DTI, MI_F32><<<grid, kBlock, 0, st>>>(va, sa, vb, sb, vo, so, rows, D, lanes_shift);
      break;
  }
  return hipGetLastError();
}

template <int DTI, int DTO>
hipError_t merge_states_chunk(int chunk, const void* v, const float* s, void* vo, float* so,
                              int64_t rows, int N, int H, int D, int lanes_shift,
                              int groups_shift, dim3 grid, hipStream_t st) {
  switch (chunk) {
    case 1:
      merge_states_kernel<DTI, DTO, 1><<<grid, kBlock, 0, st>>>(v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift);
      break;
    case 2:
      merge_states_kernel<DTI, DTO, 2><<<grid, kBlock, 0, st>>>(v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift);
      break;
    case 4:
      merge_states_kernel<DTI, DTO, 4><<<grid, kBlock, 0, st>>>(v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift);
      break;
    default:
      merge_states_kernel<DTI, DTO, 8><<<grid, kBlock, 0, st>>>(v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift);
      break;
  }
  return hipGetLastError();
}

template <int DTI>
hipError_t merge_states_out(int dt_out, int chunk, const void* v, const float* s, void* vo,
                            float* so, int64_t rows, int N, int H, int D, int lanes_shift,
                            int groups_shift, dim3 grid, hipStream_t st) {
  switch (dt_out) {
    case MI_F16:
      return merge_states_chunk<DTI, MI_F16>(chunk, v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift, grid, st);
    case MI_BF16:
      return merge_states_chunk<DTI, MI_BF16>(chunk, v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift, grid, st);
    default:
      return merge_states_chunk<DTI, MI_F32>(chunk, v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift, grid, st);
  }
}

}  // namespace

hipError_t launch_merge_state(const void* va, const float* sa, const void* vb, const float* sb,
                              void* vo, float* so, int64_t rows, int D, int dt_in, int dt_out,
                              hipStream_t st) {
  const int lanes_shift = log2_int(next_pow2(D / 8));
  const int64_t rows_per_block = kBlock >> lanes_shift;
  const dim3 grid(static_cast<unsigned>((rows + rows_per_block - 1) / rows_per_block));
  switch (dt_in) {
    case MI_F16: return merge_state_out<MI_F16>(dt_out, va, sa, vb, sb, vo, so, rows, D, lanes_shift, grid, st);
    case MI_BF16: return merge_state_out<MI_BF16>(dt_out, va, sa, vb, sb, vo, so, rows, D, lanes_shift, grid, st);
    default: return merge_state_out<MI_F32>(dt_out, va, sa, vb, sb, vo, so, rows, D, lanes_shift, grid, st);
  }
}

hipError_t launch_merge_states(const void* v, const float* s, void* vo, float* so, int64_t S,
                               int N, int H, int D, int dt_in, int dt_out, hipStream_t st) {
  const int64_t rows = S * H;
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
  const dim3 grid(static_cast<unsigned>((rows + rows_per_block - 1) / rows_per_block));
  switch (dt_in) {
    case MI_F16: return merge_states_out<MI_F16>(dt_out, chunk, v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift, grid, st);
    case MI_BF16: return merge_states_out<MI_BF16>(dt_out, chunk, v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift, grid, st);
    default: return merge_states_out<MI_F32>(dt_out, chunk, v, s, vo, so, rows, N, H, D, lanes_shift, groups_shift, grid, st);
  }
}

}  // namespace mi
