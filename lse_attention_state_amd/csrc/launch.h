// Internal launchers behind the C ABI. Arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi {

// A 1-D launch of `blocks` workgroups of `threads` lanes fits HIP's grid,
// whose size is counted in work-items in 32 bits. Launchers check this before
// launching and return hipErrorInvalidConfiguration otherwise (the C ABI
// reports MI_ERR_UNSUPPORTED), so a grid never wraps.
inline bool grid_fits(int64_t blocks, int threads) {
  return blocks >= 0 && blocks <= int64_t(0xFFFFFFFF) / threads;
}

hipError_t launch_merge_state(const void* va, const float* sa, const void* vb, const float* sb,
                              void* vo, float* so, int64_t rows, int D, int dt_in, int dt_out,
                              hipStream_t stream);

hipError_t launch_merge_states(const void* v, const float* s, void* vo, float* so, int64_t S,
                               int N, int H, int D, int dt_in, int dt_out, hipStream_t stream);

// In place: rows of positions whose mask byte is 0 are not touched (mask may be null).
hipError_t launch_merge_state_masked(void* v, float* s, const void* v_other,
                                     const float* s_other, const uint8_t* mask, int64_t rows,
                                     int H, int D, int dt, hipStream_t stream);

hipError_t launch_merge_sink(const void* v, const float* s, const float* sink, void* vo,
                             float* so, int64_t rows, int H, int D, int dt_in, int dt_out,
                             hipStream_t stream);

// Segments [indptr[p], indptr[p+1]) of v [total, H, D]; indptr null: N states per position.
// parts > 1 (indptr null): each position's states cut into `parts` slices,
// written as [S, parts, H, D] partial states (a two-level merge's first level).
hipError_t launch_merge_segments(const void* v, const float* s, const int32_t* indptr,
                                 int64_t total, int N, void* vo, float* so, int64_t S, int H,
                                 int D, int dt_in, int dt_out, hipStream_t stream, int parts = 1);

// Two-level N-state merge: the number of slices per position (1 = one level),
// and the merge itself with an fp32 workspace of S * parts * H * (D + 1) floats.
int merge_states_parts(int64_t S, int N, int H);
hipError_t launch_merge_states_two_level(const void* v, const float* s, void* vo, float* so,
                                         int64_t S, int N, int H, int D, int dt_in, int dt_out,
                                         float* ws, hipStream_t stream);

hipError_t launch_split_kv_partial(const void* q, const void* kc, const void* vc,
                                   const int32_t* page_table, int pt_stride,
                                   const int32_t* ctx_lens, int B, int Hq, int Hkv,
                                   int64_t num_phys_pages, int num_splits, float sm_scale,
                                   int kv_dtype, float* o_part, float* lse_part,
                                   hipStream_t stream, int32_t* counters = nullptr,
                                   void* o = nullptr, float* lse = nullptr, int out_dtype = -1,
                                   const float* prior_o = nullptr, const float* prior_s = nullptr,
                                   int prior_n = 0);

// Per-sequence split counts (split_indptr [B+1] on the device). counters null:
// pass 1 only; otherwise pass 1 fused with the combine.
hipError_t launch_split_kv_partial_varlen(const void* q, const void* kc, const void* vc,
                                          const int32_t* page_table, int pt_stride,
                                          const int32_t* ctx_lens, int B, int Hq, int Hkv,
                                          int64_t num_phys_pages, const int32_t* split_indptr,
                                          int total_splits, float sm_scale, int kv_dtype,
                                          float* o_part, float* lse_part, hipStream_t stream,
                                          int32_t* counters, void* o, float* lse, int out_dtype);

// Cascade prefix: chunk count and chunk length (tokens) for a shape.
void prefix_attention_plan(int R, int Hq, int Hkv, int prefix_len, int* n_chunks,
                           int* chunk_tokens);

// Cascade in two launches: the prefix chunk states into ws, then the suffix
// decode (fused) whose combine merges the splits with those chunk states.
hipError_t launch_cascade_decode(const void* q, const void* kc, const void* vc,
                                 const int32_t* prefix_pages, int prefix_len,
                                 const int32_t* suffix_table, int suffix_stride,
                                 const int32_t* suffix_lens, int R, int Hq, int Hkv,
                                 int64_t num_phys, int suffix_splits, float sm_scale,
                                 int kv_dtype, float* ws_o, float* ws_s, float* o_part,
                                 float* lse_part, int32_t* counters, void* o, float* lse,
                                 int out_dtype, hipStream_t stream);

hipError_t launch_prefix_attention(const void* q, const void* kc, const void* vc,
                                   const int32_t* prefix_pages, int prefix_len, int R, int Hq,
                                   int Hkv, int64_t num_phys, float sm_scale, int kv_dtype,
                                   float* ws_o, float* ws_s, void* v_out, float* s_out,
                                   int out_dtype, hipStream_t stream);

// Plain streaming read of `bytes` (a multiple of 16) at x; *xor_out ^= the
// XOR of all its 32-bit words.
hipError_t launch_stream_read(const void* x, int64_t bytes, uint32_t* xor_out,
                              hipStream_t stream);

}  // namespace mi
