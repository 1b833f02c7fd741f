// Cascade level 0 for gfx950: many queries against one shared prefix, as dense
// MFMA contractions ("F2 hints: merge_state, base-2 LSE merge", section 6:
// requests sharing a prefix read its KV once, the queries together form a
// matrix product, and the levels are merged afterwards).
//
// For one kv head, the query rows are the (request, query head) pairs that use
// it: row r = req * G + g reads q[req, hkv * G + g, :]. One workgroup takes a
// block of 64 rows (16 per wave) and one chunk of the prefix, and runs an
// online softmax over the chunk in tiles of 32 tokens (two pages):
//   S = Q K^T     v_mfma_f32_16x16x32 (A = Q from registers, B = K from LDS)
//   P = 2^(S*scale*log2e - m)  (rounded to the input type for the next product;
//                               the softmax denominator uses the fp32 values)
//   O += P V      v_mfma_f32_16x16x32 (A = P via LDS, B = V^T from LDS)
// K is staged in LDS row-major; V is staged transposed so that each lane's
// eight contraction values (tokens) are contiguous. Tiles are prefetched
// kTileDepth ahead in registers through per-page buffer descriptors (an absent
// page has no records and reads as zeros). Each workgroup writes its chunk's
// state (o, s) as fp32; the chunks are merged by the N-state merge kernel.
#include "common.h"
#include "launch.h"

namespace mi {
namespace {

constexpr int kD = 128;
constexpr int kPage = 16;
constexpr int kBM = 64;              // query rows per workgroup
constexpr int kBN = 32;              // prefix tokens per tile
constexpr int kThreads = 256;
constexpr int kKStride = kD + 8;     // padded LDS row (elements) of the K tile
constexpr int kVtStride = kBN + 8;   // padded LDS row (elements) of the transposed V tile
constexpr int kPStride = kBN + 8;    // padded LDS row (elements) of a wave's P tile
constexpr int kTileDepth = 3;        // tiles in flight per thread
constexpr int kMaxChunkPages = 64;   // page ids of a chunk fit one VGPR of the wave
constexpr int kBufferFlags = 0x00020000;
constexpr int kTargetBlocks = 512;   // two workgroups per compute unit

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ f32x4_t mfma16x16x32(const u32x4_t& a, const u32x4_t& b,
                                                const f32x4_t& c) {
  if constexpr (DT == MI_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Round to the 16-bit input type (nearest even) and return the bits.
template <int DT>
__device__ __forceinline__ uint16_t round16(float x) {
  if constexpr (DT == MI_BF16)
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  else
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

__device__ __forceinline__ float row16_max(float x) {
  x = __builtin_fmaxf(x, dpp<kDppQuadXor1>(x));
  x = __builtin_fmaxf(x, dpp<kDppQuadXor2>(x));
  x = __builtin_fmaxf(x, dpp<kDppRowRor4>(x));
  return __builtin_fmaxf(x, dpp<kDppRowRor8>(x));
}

template <int DT>
__global__ __launch_bounds__(kThreads) void prefix_attention_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ prefix_pages, int prefix_len,
    int n_rows, int Hq, int Hkv, int G, int64_t num_phys, int chunk_tokens, int n_chunks,
    float qk_scale_log2, float* __restrict__ ws_o, float* __restrict__ ws_s) {
  // Double-buffered K (row-major) and V (transposed) tiles; per-wave P tiles.
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][kBN * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][kD * kVtStride];
  __shared__ __attribute__((aligned(16))) uint16_t ps[4][16 * kPStride];

  // Block -> (row block, kv head, chunk). The row blocks of one (kv head,
  // chunk) get ids that are equal modulo 8, so they run on one XCD and share
  // its L2 for the chunk's K/V tiles.
  const int n_hc = Hkv * n_chunks;
  const int rb = blockIdx.x / n_hc;
  const int hc = blockIdx.x - rb * n_hc;
  const int hkv = hc / n_chunks;
  const int chunk = hc - hkv * n_chunks;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int grp = lane >> 4;

  // Q fragments (A operand): lane holds row wave*16 + l16, d = 32*k + 8*grp + [0, 8).
  u32x4_t qa[4];
  {
    const int r = rb * kBM + wave * 16 + l16;
    const int rr = r < n_rows ? r : 0;
    const int64_t qrow = static_cast<int64_t>(rr / G) * Hq + hkv * G + (rr % G);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(q + qrow * kD + 32 * k + 8 * grp);
      qa[k] = r < n_rows ? x : u32x4_t{0, 0, 0, 0};
    }
  }

  const int tok0 = chunk * chunk_tokens;
  int tok1 = tok0 + chunk_tokens;
  tok1 = tok1 < prefix_len ? tok1 : prefix_len;
  const int n_tiles = tok1 > tok0 ? (tok1 - tok0 + kBN - 1) / kBN : 0;
  const int n_pages = (prefix_len + kPage - 1) / kPage;
  const int page0 = tok0 / kPage;

  // The chunk's page ids, one per lane (a chunk spans at most 64 pages).
  const int32_t ids = (page0 + lane < n_pages) ? prefix_pages[page0 + lane] : -1;

  // Tile loads: wave w takes token rows 8w .. 8w+7 of the tile, i.e. half of
  // page w/2, so each wave's buffer descriptor is uniform. Lane l takes the
  // token pair 8w + 2(l%4), +1 at d = 8(l/4); a load instruction covers four
  // whole 256-byte rows, and each lane can write V^T as packed token pairs.
  const int pr = lane & 3;
  const int c8 = (lane >> 2) * 8;
  const int row0 = (wave & 1) * 8 + 2 * pr;            // token row within the page
  const int lane_bytes = (row0 * kD + c8) * 2;
  const int64_t tile_elems = static_cast<int64_t>(kPage) * kD;
  u32x4_t kbuf[kTileDepth][2], vbuf[kTileDepth][2];
  auto issue = [&](int t, int j) {
    const int pl = 2 * t + (wave >> 1);                 // page index within the chunk
    const int32_t phys = __builtin_amdgcn_readlane(ids, pl & 63);
    const bool ok = t < n_tiles && page0 + pl < n_pages && phys >= 0 && phys < num_phys;
    const int64_t base = (static_cast<int64_t>(ok ? phys : 0) * Hkv + hkv) * tile_elems;
    const int records = ok ? static_cast<int>(tile_elems * 2) : 0;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kc + base), 0, records, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vc + base), 0, records, kBufferFlags);
    kbuf[j][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, lane_bytes, 0, 0));
    kbuf[j][1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, lane_bytes + kD * 2, 0, 0));
    vbuf[j][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, lane_bytes, 0, 0));
    vbuf[j][1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, lane_bytes + kD * 2, 0, 0));
  };

  // Stage tile t (registers slot j) into LDS buffer `buf`; tokens at or past
  // the chunk end are zero in V (their scores are masked separately).
  const int tk = 8 * wave + 2 * pr;                     // token pair within the tile
  auto stage = [&](int t, int j, int buf) {
    const int ttok = tok0 + t * kBN;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<u32x4_t*>(&ks[buf][(tk + h) * kKStride + c8]) = kbuf[j][h];
    const bool v0 = ttok + tk < tok1;
    const bool v1 = ttok + tk + 1 < tok1;
    const u32x4_t a = v0 ? vbuf[j][0] : u32x4_t{0, 0, 0, 0};
    const u32x4_t b = v1 ? vbuf[j][1] : u32x4_t{0, 0, 0, 0};
    uint32_t* vtw = reinterpret_cast<uint32_t*>(vt[buf]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = a[i], y = b[i];
      vtw[((c8 + 2 * i) * kVtStride + tk) / 2] = (x & 0xffffu) | (y << 16);
      vtw[((c8 + 2 * i + 1) * kVtStride + tk) / 2] = (x >> 16) | (y & 0xffff0000u);
    }
  };

  f32x4_t o[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) o[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m[4], lsum[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    m[e] = -kInf;
    lsum[e] = 0.0f;
  }

  auto compute = [&](int t, int buf) {
    const int ttok = tok0 + t * kBN;
    // S = Q K^T for the wave's 16 rows and the tile's 32 tokens (two 16-column tiles).
    f32x4_t s[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) s[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const u32x4_t kb = *reinterpret_cast<const u32x4_t*>(
            &ks[buf][(16 * c + l16) * kKStride + 32 * k + 8 * grp]);
        s[c] = mfma16x16x32<DT>(qa[k], kb, s[c]);
      }
    }
    // Online softmax for the lane's rows 4*grp + e (columns 16c + l16).
    uint16_t pbits[2][4];
    float alpha[4];
    bool moved = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x0 = s[0][e] * qk_scale_log2;
      float x1 = s[1][e] * qk_scale_log2;
      x0 = ttok + l16 < tok1 ? x0 : -kInf;
      x1 = ttok + 16 + l16 < tok1 ? x1 : -kInf;
      const float mn = __builtin_fmaxf(m[e], row16_max(__builtin_fmaxf(x0, x1)));
      const float mu = mn == -kInf ? 0.0f : mn;
      alpha[e] = __builtin_amdgcn_exp2f(m[e] - mu);
      moved |= mn != m[e];
      // The denominator takes the fp32 weights; only the P V product uses the
      // weights rounded to the input type (the LSE stays exact to fp32).
      const float p0 = __builtin_amdgcn_exp2f(x0 - mu);
      const float p1 = __builtin_amdgcn_exp2f(x1 - mu);
      pbits[0][e] = round16<DT>(p0);
      pbits[1][e] = round16<DT>(p1);
      lsum[e] = lsum[e] * alpha[e] + (p0 + p1);
      m[e] = mn;
    }
    if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c][e] *= alpha[e];
    }
    // P to LDS (row-major per wave), read back as the A operand of P V.
    uint16_t* pw = ps[wave];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pw[(4 * grp + e) * kPStride + l16] = pbits[0][e];
      pw[(4 * grp + e) * kPStride + 16 + l16] = pbits[1][e];
    }
    const u32x4_t pa = *reinterpret_cast<const u32x4_t*>(pw + l16 * kPStride + 8 * grp);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const u32x4_t vb = *reinterpret_cast<const u32x4_t*>(
          &vt[buf][(16 * c + l16) * kVtStride + 8 * grp]);
      o[c] = mfma16x16x32<DT>(pa, vb, o[c]);
    }
  };

  // Pipeline: registers hold tiles t+1 .. t+kTileDepth; tile t+1 is staged
  // into the other LDS buffer while tile t is computed; one barrier per tile.
  // The loop body is unconditional: tiles past the chunk end load zeros (no
  // records) and have every score masked, so they change nothing, and the
  // compiler can keep exact load counts across iterations.
#pragma unroll
  for (int j = 0; j < kTileDepth; ++j) {
    issue(j, j);
    __builtin_amdgcn_sched_barrier(0);
  }
  stage(0, 0, 0);
  issue(kTileDepth, 0);
  __syncthreads();
  const int iters = (n_tiles + kTileDepth - 1) / kTileDepth * kTileDepth;
  for (int base = 0; base < iters; base += kTileDepth) {
#pragma unroll
    for (int j = 0; j < kTileDepth; ++j) {
      const int t = base + j;
      const int jn = (j + 1) % kTileDepth;   // register slot of tile t+1
      stage(t + 1, jn, (t + 1) & 1);
      issue(t + 1 + kTileDepth, jn);
      compute(t, t & 1);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Finalise the chunk state of the lane's rows 4*grp + e, columns 16c + l16.
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float l = row16_sum(lsum[e]);
    const float inv = guarded_inv(l);
    const int r = rb * kBM + wave * 16 + 4 * grp + e;
    if (r >= n_rows) continue;
    const int64_t qrow = static_cast<int64_t>(r / G) * Hq + hkv * G + (r % G);
    const int64_t at = qrow * n_chunks + chunk;
    float* out = ws_o + at * kD + l16;
#pragma unroll
    for (int c = 0; c < 8; ++c) out[16 * c] = o[c][e] * inv;
    if (l16 == 0) ws_s[at] = l > 0.0f ? m[e] + hw_log2(l) : -kInf;
  }
}

}  // namespace

void prefix_attention_plan(int R, int Hq, int Hkv, int prefix_len, int* n_chunks,
                           int* chunk_tokens) {
  const int G = Hq / Hkv;
  const int n_rb = (R * G + kBM - 1) / kBM;
  const int max_chunks = prefix_len > 0 ? (prefix_len + kBN - 1) / kBN : 1;
  int c = kTargetBlocks / (n_rb * Hkv);
  c = c < 1 ? 1 : (c > max_chunks ? max_chunks : c);
  int tokens = prefix_len > 0 ? (prefix_len + c - 1) / c : kBN;
  tokens = (tokens + kBN - 1) / kBN * kBN;
  if (tokens > kMaxChunkPages * kPage) tokens = kMaxChunkPages * kPage;
  *chunk_tokens = tokens;
  *n_chunks = prefix_len > 0 ? (prefix_len + tokens - 1) / tokens : 1;
}

hipError_t launch_prefix_attention(const void* q, const void* kc, const void* vc,
                                   const int32_t* prefix_pages, int prefix_len, int R, int Hq,
                                   int Hkv, int64_t num_phys, float sm_scale, int kv_dtype,
                                   float* ws_o, float* ws_s, void* v_out, float* s_out,
                                   int out_dtype, hipStream_t st) {
  int n_chunks, chunk_tokens;
  prefix_attention_plan(R, Hq, Hkv, prefix_len, &n_chunks, &chunk_tokens);
  const int G = Hq / Hkv;
  const int n_rows = R * G;
  const int n_rb = (n_rows + kBM - 1) / kBM;
  const dim3 grid(static_cast<unsigned>(n_rb * Hkv * n_chunks));
  const float scale = static_cast<float>(static_cast<double>(sm_scale) * 1.4426950408889634);
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(kc);
  const uint16_t* v16 = static_cast<const uint16_t*>(vc);
  if (kv_dtype == MI_BF16)
    prefix_attention_kernel<MI_BF16><<<grid, kThreads, 0, st>>>(
        q16, k16, v16, prefix_pages, prefix_len, n_rows, Hq, Hkv, G, num_phys, chunk_tokens,
        n_chunks, scale, ws_o, ws_s);
  else
    prefix_attention_kernel<MI_F16><<<grid, kThreads, 0, st>>>(
        q16, k16, v16, prefix_pages, prefix_len, n_rows, Hq, Hkv, G, num_phys, chunk_tokens,
        n_chunks, scale, ws_o, ws_s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Merge the chunk states: ws [R*Hq, n_chunks, 1, D] -> [R*Hq, 1, D].
  return launch_merge_states(ws_o, ws_s, v_out, s_out, static_cast<int64_t>(R) * Hq, n_chunks,
                             1, kD, MI_F32, out_dtype, st);
}

}  // namespace mi
