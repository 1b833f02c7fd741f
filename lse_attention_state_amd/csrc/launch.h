// Internal launchers behind the C ABI. Arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi {

hipError_t launch_merge_state(const void* va, const float* sa, const void* vb, const float* sb,
                              void* vo, float* so, int64_t rows, int D, int dt_in, int dt_out,
                              hipStream_t stream);

hipError_t launch_merge_states(const void* v, const float* s, void* vo, float* so, int64_t S,
                               int N, int H, int D, int dt_in, int dt_out, hipStream_t stream);

hipError_t launch_split_kv_partial(const void* q, const void* kc, const void* vc,
                                   const int32_t* page_table, int pt_stride,
                                   const int32_t* ctx_lens, int B, int Hq, int Hkv,
                                   int64_t num_phys_pages, int num_splits, float sm_scale,
                                   int kv_dtype, float* o_part, float* lse_part,
                                   hipStream_t stream, int32_t* counters = nullptr,
                                   void* o = nullptr, float* lse = nullptr, int out_dtype = -1);

// Cascade prefix: chunk count and chunk length (tokens) for a shape.
void prefix_attention_plan(int R, int Hq, int Hkv, int prefix_len, int* n_chunks,
                           int* chunk_tokens);

hipError_t launch_prefix_attention(const void* q, const void* kc, const void* vc,
                                   const int32_t* prefix_pages, int prefix_len, int R, int Hq,
                                   int Hkv, int64_t num_phys, float sm_scale, int kv_dtype,
                                   float* ws_o, float* ws_s, void* v_out, float* s_out,
                                   int out_dtype, hipStream_t stream);

}  // namespace mi
