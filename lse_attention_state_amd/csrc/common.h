// Device helpers for the gfx950 kernels: 16-byte vector loads/stores of
// 8-element chunks, fp16/bf16 <-> fp32 conversion, the empty-state guards,
// and wave64 cross-lane operations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mi.h"

namespace mi {

constexpr float kInf = __builtin_inff();

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- guards

// "FlashAttention's empty-row LSE", section 2.2: NaN and +inf fold to -inf.
__device__ __forceinline__ float sanitize_lse(float s) {
  return (s != s || s == kInf) ? -kInf : s;
}

// Weight 2^(s - m) with the max-based NaN guard ("F2 hints", section 5):
// when s and m are both -inf, s - m is NaN and fmaxf(NaN, -inf) = -inf, so the
// weight is 0 instead of NaN. v_exp_f32 is the hardware 2^x.
__device__ __forceinline__ float guarded_exp2(float diff) {
  return __builtin_amdgcn_exp2f(__builtin_fmaxf(diff, -kInf));
}

__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

// 1/Z, or 0 when Z is 0 or NaN ("FlashAttention's empty-row LSE", section 4.1).
__device__ __forceinline__ float guarded_inv(float z) {
  return (z > 0.0f) ? __builtin_amdgcn_rcpf(z) : 0.0f;
}

// ---------------------------------------------------------------- conversions
//
// Reinterpretations take a scalar by value: applying __builtin_bit_cast
// directly to an ext-vector element (v[i]) reads element 0 with this compiler,
// so vector elements are always copied into a scalar first.

__device__ __forceinline__ half2_t as_half2(uint32_t w) { return __builtin_bit_cast(half2_t, w); }
__device__ __forceinline__ bf162_t as_bf162(uint32_t w) { return __builtin_bit_cast(bf162_t, w); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_lo(uint32_t w) { return static_cast<float>(as_half2(w).x); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return static_cast<float>(as_half2(w).y); }

// Round-to-nearest-even packing of two fp32 values.
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  half2_t h = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf162_t h = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, h);
}

// ---------------------------------------------------------------- 8-element chunks

// Element type of a dtype code, for byte-size arithmetic.
template <int DT> struct Elem;
template <> struct Elem<MI_F16> { static constexpr int bytes = 2; };
template <> struct Elem<MI_BF16> { static constexpr int bytes = 2; };
template <> struct Elem<MI_F32> { static constexpr int bytes = 4; };

// Load 8 consecutive elements starting at element offset `off` as fp32.
// 16-bit types: one 16-byte load; fp32: two 16-byte loads. The loads carry the
// non-temporal hint: merge inputs are streamed once (measured: +10-18% HBM
// throughput for the two merge kernels on MI355X).
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t off, float (&x)[8]) {
  if constexpr (DT == MI_F32) {
    const float4_t* p = reinterpret_cast<const float4_t*>(static_cast<const float*>(base) + off);
    const float4_t a = __builtin_nontemporal_load(p);
    const float4_t b = __builtin_nontemporal_load(p + 1);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
    const u32x4_t w = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(base) + off));
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
}

// The same load in two steps: the raw words (two 16-byte loads for fp32, one
// for 16-bit types), then their conversion to fp32. Kernels that keep many
// loads in flight issue all raw loads, place a scheduling barrier, and only
// then convert, so no conversion is scheduled between the loads (which would
// make the wave wait for one of them early).
struct Raw8 {
  u32x4_t a, b;
};

template <int DT>
__device__ __forceinline__ Raw8 load8_raw(const void* base, int64_t off) {
  Raw8 r;
  if constexpr (DT == MI_F32) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(static_cast<const float*>(base) + off);
    r.a = __builtin_nontemporal_load(p);
    r.b = __builtin_nontemporal_load(p + 1);
  } else {
    r.a = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(base) + off));
    r.b = u32x4_t{0, 0, 0, 0};
  }
  return r;
}

template <int DT>
__device__ __forceinline__ void unpack8_raw(const Raw8& r, float (&x)[8]) {
  if constexpr (DT == MI_F32) {
    // Cast whole vectors: a bit_cast of a single ext-vector element has been
    // compiled as a read of element 0.
    const float4_t fa = __builtin_bit_cast(float4_t, r.a);
    const float4_t fb = __builtin_bit_cast(float4_t, r.b);
    x[0] = fa.x; x[1] = fa.y; x[2] = fa.z; x[3] = fa.w;
    x[4] = fb.x; x[5] = fb.y; x[6] = fb.z; x[7] = fb.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == MI_F16) {
        x[2 * i] = f16_lo(r.a[i]);
        x[2 * i + 1] = f16_hi(r.a[i]);
      } else {
        x[2 * i] = bf16_lo(r.a[i]);
        x[2 * i + 1] = bf16_hi(r.a[i]);
      }
    }
  }
}

// Store of 8 elements rounded to DT. kStream: with the non-temporal hint, for
// outputs a streaming kernel writes once and does not read back (measured on
// MI355X for the two-state merge: its dirty output no longer lingers in the
// last-level cache to be written back during the next kernel, which made that
// kernel 7-8% slower). Which policy a kernel uses is measured per kernel.
template <int DT, bool kStream = false>
__device__ __forceinline__ void store8(void* base, int64_t off, const float (&x)[8]) {
  if constexpr (kStream) {
    if constexpr (DT == MI_F32) {
      float4_t* p = reinterpret_cast<float4_t*>(static_cast<float*>(base) + off);
      __builtin_nontemporal_store(float4_t{x[0], x[1], x[2], x[3]}, p);
      __builtin_nontemporal_store(float4_t{x[4], x[5], x[6], x[7]}, p + 1);
    } else {
      u32x4_t w;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (DT == MI_F16) ? pack_f16(x[2 * i], x[2 * i + 1]) : pack_bf16(x[2 * i], x[2 * i + 1]);
      __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(base) + off));
    }
    return;
  }
  if constexpr (DT == MI_F32) {
    float4_t* p = reinterpret_cast<float4_t*>(static_cast<float*>(base) + off);
    p[0] = float4_t{x[0], x[1], x[2], x[3]};
    p[1] = float4_t{x[4], x[5], x[6], x[7]};
  } else {
    u32x4_t w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (DT == MI_F16) ? pack_f16(x[2 * i], x[2 * i + 1]) : pack_bf16(x[2 * i], x[2 * i + 1]);
    *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(base) + off) = w;
  }
}

// ---------------------------------------------------------------- cross-lane

// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;  // rotate right by 4 within a row of 16
constexpr int kDppRowRor8 = 0x128;  // rotate right by 8 within a row of 16

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of each row; every lane of the row receives the sum.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowRor4>(x);
  x += dpp<kDppRowRor8>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor(float x, int mask) {
  const int lane = __lane_id();
  return __builtin_bit_cast(
      float, __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __builtin_bit_cast(int, x)));
}

}  // namespace mi
