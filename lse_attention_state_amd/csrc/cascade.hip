// Cascade level 0 for gfx950: many queries against one shared prefix, as dense
// MFMA contractions ("F2 hints: merge_state, base-2 LSE merge", section 6:
// requests sharing a prefix read its KV once, the queries together form a
// matrix product, and the levels are merged afterwards).
//
// For one kv head, the query rows are the (request, query head) pairs that use
// it: row r = req * G + g reads q[req, hkv * G + g, :]. One workgroup takes a
// block of 64 rows (one 16-row MFMA tile per wave) and one chunk of the
// prefix, and runs an online softmax over the chunk in tiles of 32 tokens
// (two pages). Two workgroups share a compute unit (two waves per SIMD), so
// one wave's softmax arithmetic overlaps the other's matrix products.
// Everything is computed transposed, so that the softmax weights never leave
// registers:
//   S^T = K Q^T    v_mfma_f32_16x16x32: A = K (16 tokens x 32 d) from LDS,
//                  B = Q^T from registers; lane (l16, grp) receives the scores
//                  of row l16 for tokens 4grp+e and 16+4grp+e (e < 4)
//   P^T = 2^(S^T*scale*log2e - m), rounded to the input type: those eight
//                  weights are exactly the lane's B operand of the next product
//                  when its contraction slot grp holds those eight tokens
//   O^T += V^T P^T v_mfma_f32_16x16x32: A = V^T (16 d x 32 tokens), read from
//                  the row-major V tile with gfx950's transposing LDS read
//                  (ds_read_b64_tr_b16: within each group of 16 lanes, lane j
//                  receives element j%4 of the 8 bytes read by lanes j/4,
//                  4+j/4, 8+j/4 and 12+j/4, so lanes that read 4 d values of
//                  4 token rows hand each lane 4 tokens at one d)
// The softmax denominator sums the fp32 weights, so the LSE is exact to fp32;
// only the P V product uses the rounded weights. The running max of a row is
// shared by the four lanes that hold it; it is raised only when a score passes
// it by more than kRescaleSlack (rare after the first tile), which is when the
// four lanes compare their maxima.
//
// K and V tiles are both staged row-major with 288-byte rows, the stride
// measured free of bank conflicts on gfx950 for the K reads (16 rows x 16
// bytes per ds_read_b128; 272 bytes measured 1.7x slower, 256 bytes 6.5x).
// (An earlier form staged V transposed with v_perm and scattered 4-byte
// writes; the transposing read removes that work and runs 6% faster.)
// Tiles are prefetched kDepth ahead in registers through per-page buffer
// descriptors; an absent page reads as zeros and contributes no tokens. Each workgroup writes its chunk's state
// (o, s) as fp32; the chunks are merged by the N-state merge kernel.
#include "common.h"
#include "launch.h"

namespace mi {
namespace {

constexpr int kD = 128;
constexpr int kPage = 16;
constexpr int kRowTiles = 1;               // 16-row MFMA tiles per wave
constexpr int kBM = 4 * 16 * kRowTiles;    // query rows per workgroup
constexpr int kBN = 32;                    // prefix tokens per tile
constexpr int kThreads = 256;
constexpr int kKStride = kD + 16;          // LDS row (elements) of the K tile: 288 bytes
constexpr int kVStride = kD + 16;          // LDS row (elements) of the V tile: 288 bytes
constexpr int kDepth = 2;                  // tiles in flight per thread (2 measured faster than 4 or 6)
constexpr int kMaxChunkPages = 64;         // page ids of a chunk fit one VGPR of the wave
constexpr int kBufferFlags = 0x00020000;
constexpr float kRescaleSlack = 8.0f;
constexpr int kTargetBlocks = 512;        // two workgroups per compute unit

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

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

// Two fp32 values rounded to the 16-bit input type (nearest even), packed.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return DT == MI_BF16 ? pack_bf16(a, b) : pack_f16(a, b);
}

template <int DT>
__global__ __launch_bounds__(kThreads, 2) void prefix_attention_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ prefix_pages, int prefix_len,
    int n_rows, int Hq, int Hkv, int G, int64_t num_phys, int chunk_tokens, int n_chunks,
    float qk_scale_log2, float* __restrict__ ws_o, float* __restrict__ ws_s) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][kBN * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][kBN * kVStride];

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

  // Q^T fragments (B operand): lane holds row l16 of row tile r, d = 32k + 8grp + [0, 8).
  u32x4_t qb[kRowTiles][4];
#pragma unroll
  for (int r = 0; r < kRowTiles; ++r) {
    const int row = rb * kBM + wave * (16 * kRowTiles) + 16 * r + l16;
    const int rr = row < n_rows ? row : 0;
    const int64_t qrow = static_cast<int64_t>(rr / G) * Hq + hkv * G + (rr % G);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(q + qrow * kD + 32 * k + 8 * grp);
      qb[r][k] = row < n_rows ? x : u32x4_t{0, 0, 0, 0};
    }
  }

  const int tok0 = chunk * chunk_tokens;
  int tok1 = tok0 + chunk_tokens;
  tok1 = tok1 < prefix_len ? tok1 : prefix_len;
  const int n_tiles = tok1 > tok0 ? (tok1 - tok0 + kBN - 1) / kBN : 0;
  const int n_pages = (prefix_len + kPage - 1) / kPage;
  const int page0 = tok0 / kPage;

  // The chunk's page ids, one per lane (a chunk spans at most 64 pages), and
  // which of them hold tokens of this chunk: bit pl of ok_pages is set when
  // chunk page pl exists, lies inside the chunk's tiles and has a valid id, so
  // every later validity test is a scalar bit test.
  const int32_t ids = (page0 + lane < n_pages) ? prefix_pages[page0 + lane] : -1;
  const uint64_t ok_pages = __builtin_amdgcn_ballot_w64(
      page0 + lane < n_pages && lane < 2 * n_tiles && ids >= 0 && ids < num_phys);
  auto page_ok = [&](int pl, int32_t) { return pl < 64 && ((ok_pages >> pl) & 1) != 0; };

  // Staging: thread (p = tid/16, c = tid%16) takes tile tokens 2p, 2p+1 at
  // d = 8c of both K and V (its wave covers one page: p/8 = wave/2).
  const int kp = tid >> 4, kc8 = (tid & 15) * 8;
  const int k_lane_bytes = ((2 * (kp & 7)) * kD + kc8) * 2;
  const int64_t tile_elems = static_cast<int64_t>(kPage) * kD;
  u32x4_t kbuf[kDepth][2], vbuf[kDepth][2];
  bool vok[kDepth];
  bool vfull[kDepth];  // the whole tile is valid (uniform)
  auto issue = [&](int t, int j) {
    {  // K: the wave's page
      const int pl = 2 * t + (wave >> 1);
      const int32_t phys = __builtin_amdgcn_readlane(ids, pl & 63);
      const bool ok = page_ok(pl, phys);
      const int64_t base = (static_cast<int64_t>(ok ? phys : 0) * Hkv + hkv) * tile_elems;
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(kc + base), 0, ok ? static_cast<int>(tile_elems * 2) : 0, kBufferFlags);
      kbuf[j][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, k_lane_bytes, 0, 0));
      kbuf[j][1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, k_lane_bytes + kD * 2, 0, 0));
    }
    {  // V: the wave's page, rows as for K
      const int pl = 2 * t + (wave >> 1);
      const int32_t phys = __builtin_amdgcn_readlane(ids, pl & 63);
      const bool ok = page_ok(pl, phys);
      vok[j] = ok;
      vfull[j] = page_ok(2 * t, __builtin_amdgcn_readlane(ids, (2 * t) & 63)) &&
                 page_ok(2 * t + 1, __builtin_amdgcn_readlane(ids, (2 * t + 1) & 63)) &&
                 tok0 + (t + 1) * kBN <= tok1;
      const int64_t base = (static_cast<int64_t>(ok ? phys : 0) * Hkv + hkv) * tile_elems;
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(vc + base), 0, ok ? static_cast<int>(tile_elems * 2) : 0, kBufferFlags);
      vbuf[j][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, k_lane_bytes, 0, 0));
      vbuf[j][1] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, k_lane_bytes + kD * 2, 0, 0));
    }
  };

  // Stage tile t (register slot j) into LDS buffer `buf`, K and V row-major.
  // V of tokens at or past the chunk end or on an absent page is written as
  // zero (their scores are masked as well, and 0 * NaN must not reach O).
  auto stage = [&](int t, int j, int buf) {
    *reinterpret_cast<u32x4_t*>(&ks[buf][(2 * kp) * kKStride + kc8]) = kbuf[j][0];
    *reinterpret_cast<u32x4_t*>(&ks[buf][(2 * kp + 1) * kKStride + kc8]) = kbuf[j][1];
    u32x4_t a = vbuf[j][0], b = vbuf[j][1];
    if (!vfull[j]) {  // the chunk's last tile, or an absent page (already zeros)
      const int ttok = tok0 + t * kBN;
      a = (vok[j] && ttok + 2 * kp < tok1) ? a : u32x4_t{0, 0, 0, 0};
      b = (vok[j] && ttok + 2 * kp + 1 < tok1) ? b : u32x4_t{0, 0, 0, 0};
    }
    *reinterpret_cast<u32x4_t*>(&vs[buf][(2 * kp) * kVStride + kc8]) = a;
    *reinterpret_cast<u32x4_t*>(&vs[buf][(2 * kp + 1) * kVStride + kc8]) = b;
  };

  f32x4_t o[kRowTiles][8];
  // m: reference max of a row (base 2), mu: m or 0 while m = -inf (the value
  // subtracted before exp2), gap: how far above mu a score may go before m is
  // raised (kRescaleSlack, or -inf while m = -inf).
  float m[kRowTiles], mu[kRowTiles], gap[kRowTiles], lsum[kRowTiles];
#pragma unroll
  for (int r = 0; r < kRowTiles; ++r) {
#pragma unroll
    for (int c = 0; c < 8; ++c) o[r][c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m[r] = -kInf;
    mu[r] = 0.0f;
    gap[r] = -kInf;
    lsum[r] = 0.0f;
  }

  auto compute = [&](int t, int buf) {
    const int ttok = tok0 + t * kBN;
    // S^T: token tile c (tokens 16c..16c+15) x the wave's row tiles.
    f32x4_t s[kRowTiles][2];
#pragma unroll
    for (int r = 0; r < kRowTiles; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c) s[r][c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // All K operands are read before the products, likewise the V^T operands
    // below, which are read before the softmax arithmetic so that their LDS
    // latency overlaps it.
    u32x4_t ka[4][2];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        ka[k][c] = *reinterpret_cast<const u32x4_t*>(
            &ks[buf][(16 * c + l16) * kKStride + 32 * k + 8 * grp]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int r = 0; r < kRowTiles; ++r) s[r][c] = mfma16x16x32<DT>(ka[k][c], qb[r][k], s[r][c]);
    // V^T operand of d block c: lane (l16, grp) needs d = 16c + l16 at tokens
    // 4grp..4grp+3 and 16+4grp..16+4grp+3; a transposing read in which lane s
    // of each 16-lane group reads 4 d values of token row s/4 gives lane j the
    // 4 token values at d column j.
    u32x4_t va[8];
    const int tr_row = 4 * grp + (l16 >> 2);
    const int tr_col = 4 * (l16 & 3);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(&vs[buf][tr_row * kVStride + 16 * c + tr_col]));
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(&vs[buf][(16 + tr_row) * kVStride + 16 * c + tr_col]));
      const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo);
      const u32x2_t h2 = __builtin_bit_cast(u32x2_t, hi);
      va[c] = u32x4_t{l2.x, l2.y, h2.x, h2.y};
    }
    __builtin_amdgcn_sched_barrier(0);
    // y = score * scale * log2(e) - mu, one FMA per score. Tokens at or past
    // the chunk end, or on an absent page, get y = -inf; only the chunk's last
    // tile (or one with an absent page) needs the masks.
    const bool full = tok0 + (t + 1) * kBN <= tok1 &&
                      page_ok(2 * t, __builtin_amdgcn_readlane(ids, (2 * t) & 63)) &&
                      page_ok(2 * t + 1, __builtin_amdgcn_readlane(ids, (2 * t + 1) & 63));
    float y[kRowTiles][8];
    auto make_y = [&](int r) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) y[r][4 * c + e] = __builtin_fmaf(s[r][c][e], qk_scale_log2, -mu[r]);
      if (!full) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const bool pg = page_ok(2 * t + c, __builtin_amdgcn_readlane(ids, (2 * t + c) & 63));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool in = pg && ttok + 16 * c + 4 * grp + e < tok1;
            y[r][4 * c + e] = in ? y[r][4 * c + e] : -kInf;
          }
        }
      }
    };
    bool need = false;
    float ymax[kRowTiles];
#pragma unroll
    for (int r = 0; r < kRowTiles; ++r) {
      make_y(r);
      ymax[r] = y[r][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) ymax[r] = __builtin_fmaxf(ymax[r], y[r][i]);
      need |= ymax[r] > gap[r];
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      // Raise the row maxima: the four lanes of a row agree on the new max.
#pragma unroll
      for (int r = 0; r < kRowTiles; ++r) {
        float mx = __builtin_fmaxf(m[r], ymax[r] + mu[r]);
        mx = __builtin_fmaxf(mx, shfl_xor(mx, 16));
        mx = __builtin_fmaxf(mx, shfl_xor(mx, 32));
        const float alpha = mx > m[r] ? __builtin_amdgcn_exp2f(m[r] - mx) : 1.0f;
        m[r] = mx;
        mu[r] = mx == -kInf ? 0.0f : mx;
        gap[r] = mx == -kInf ? -kInf : kRescaleSlack;
        lsum[r] *= alpha;
#pragma unroll
        for (int c = 0; c < 8; ++c) o[r][c] *= alpha;
        make_y(r);
      }
    }
    // P^T as the B operand: slot grp holds tokens 4grp..4grp+3, 16+4grp..16+4grp+3.
    u32x4_t pb[kRowTiles];
#pragma unroll
    for (int r = 0; r < kRowTiles; ++r) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = __builtin_amdgcn_exp2f(y[r][i]);
        lsum[r] += p[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[r][i] = pack2<DT>(p[2 * i], p[2 * i + 1]);
    }
    // O^T += V^T P^T over the eight 16-wide d tiles.
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int r = 0; r < kRowTiles; ++r) o[r][c] = mfma16x16x32<DT>(va[c], pb[r], o[r][c]);
  };

  // Pipeline: registers hold tiles t+1 .. t+kDepth; tile t+1 is staged into
  // the other LDS buffer while tile t is computed; one barrier per tile. The
  // loop body is unconditional: tiles past the chunk end load zeros (no
  // records, or a masked page) and have every score masked, so they change
  // nothing, and the compiler keeps exact load counts across iterations.
#pragma unroll
  for (int j = 0; j < kDepth; ++j) {
    issue(j, j);
    __builtin_amdgcn_sched_barrier(0);
  }
  stage(0, 0, 0);
  issue(kDepth, 0);
  __syncthreads();
  const int iters = (n_tiles + kDepth - 1) / kDepth * kDepth;
  for (int base = 0; base < iters; base += kDepth) {
#pragma unroll
    for (int j = 0; j < kDepth; ++j) {
      const int t = base + j;
      const int jn = (j + 1) % kDepth;   // register slot of tile t+1
      stage(t + 1, jn, (t + 1) & 1);
      issue(t + 1 + kDepth, jn);
      compute(t, t & 1);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Finalise the chunk state of row l16 of each row tile: lane (l16, grp)
  // holds d = 16c + 4grp + e; the denominator is summed over the four lanes.
#pragma unroll
  for (int r = 0; r < kRowTiles; ++r) {
    float l = lsum[r];
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    const float inv = guarded_inv(l);
    const int row = rb * kBM + wave * (16 * kRowTiles) + 16 * r + l16;
    if (row >= n_rows) continue;
    const int64_t qrow = static_cast<int64_t>(row / G) * Hq + hkv * G + (row % G);
    const int64_t at = qrow * n_chunks + chunk;
    float* out = ws_o + at * kD + 4 * grp;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      *reinterpret_cast<f32x4_t*>(out + 16 * c) = o[r][c] * inv;
    if (grp == 0) ws_s[at] = l > 0.0f ? m[r] + hw_log2(l) : -kInf;
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

hipError_t launch_prefix_chunks(const void* q, const void* kc, const void* vc,
                                const int32_t* prefix_pages, int prefix_len, int R, int Hq,
                                int Hkv, int64_t num_phys, float sm_scale, int kv_dtype,
                                float* ws_o, float* ws_s, hipStream_t st) {
  int n_chunks, chunk_tokens;
  prefix_attention_plan(R, Hq, Hkv, prefix_len, &n_chunks, &chunk_tokens);
  const int G = Hq / Hkv;
  const int n_rows = R * G;
  const int n_rb = (n_rows + kBM - 1) / kBM;
  const int64_t blocks = int64_t(n_rb) * Hkv * n_chunks;
  if (!grid_fits(blocks, kThreads)) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(blocks));
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
  return hipGetLastError();
}

hipError_t launch_prefix_attention(const void* q, const void* kc, const void* vc,
                                   const int32_t* prefix_pages, int prefix_len, int R, int Hq,
                                   int Hkv, int64_t num_phys, float sm_scale, int kv_dtype,
                                   float* ws_o, float* ws_s, void* v_out, float* s_out,
                                   int out_dtype, hipStream_t st) {
  hipError_t e = launch_prefix_chunks(q, kc, vc, prefix_pages, prefix_len, R, Hq, Hkv, num_phys,
                                      sm_scale, kv_dtype, ws_o, ws_s, st);
  if (e != hipSuccess) return e;
  int n_chunks, chunk_tokens;
  prefix_attention_plan(R, Hq, Hkv, prefix_len, &n_chunks, &chunk_tokens);
  // Merge the chunk states: ws [R*Hq, n_chunks, 1, D] -> [R*Hq, 1, D].
  return launch_merge_states(ws_o, ws_s, v_out, s_out, static_cast<int64_t>(R) * Hq, n_chunks,
                             1, kD, MI_F32, out_dtype, st);
}

hipError_t launch_cascade_decode(const void* q, const void* kc, const void* vc,
                                 const int32_t* prefix_pages, int prefix_len,
                                 const int32_t* suffix_table, int suffix_stride,
                                 const int32_t* suffix_lens, int R, int Hq, int Hkv,
                                 int64_t num_phys, int suffix_splits, float sm_scale,
                                 int kv_dtype, float* ws_o, float* ws_s, float* o_part,
                                 float* lse_part, int32_t* counters, void* o, float* lse,
                                 int out_dtype, hipStream_t st) {
  hipError_t e = launch_prefix_chunks(q, kc, vc, prefix_pages, prefix_len, R, Hq, Hkv, num_phys,
                                      sm_scale, kv_dtype, ws_o, ws_s, st);
  if (e != hipSuccess) return e;
  int n_chunks, chunk_tokens;
  prefix_attention_plan(R, Hq, Hkv, prefix_len, &n_chunks, &chunk_tokens);
  // The suffix level, whose combine also merges each row's prefix chunk states.
  return launch_split_kv_partial(q, kc, vc, suffix_table, suffix_stride, suffix_lens, R, Hq, Hkv,
                                 num_phys, suffix_splits, sm_scale, kv_dtype, o_part, lse_part,
                                 st, counters, o, lse, out_dtype, ws_o, ws_s, n_chunks);
}

}  // namespace mi
