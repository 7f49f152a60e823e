// ssm_math.hpp -- device-side scalar helpers for the S6 kernels (gfx950).
//
// Transcendentals use the hardware base-2 units (v_exp_f32, v_log_f32,
// v_rcp_f32); the scan step itself needs one v_exp_f32 per (element, state):
// Abar = exp(Delta*A) = exp2(Delta * (A*log2 e)), with A*log2 e formed once
// per channel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// ln(1 + w) for w in [0, 1].  Below 1/16 an 8-term Taylor series (truncation
// below 2^-34 relative).  Above, the hardware log of u = fl(1 + w), whose
// argument is then far enough from 1 for full relative precision, times
// w / (u - 1) to undo the rounding of u (u - 1 is exact).
__device__ __forceinline__ float log1p_unit(float w) {
  if (w < 0.0625f) {
    float p = -1.0f / 8.0f;
    p = __builtin_fmaf(p, w, 1.0f / 7.0f);
    p = __builtin_fmaf(p, w, -1.0f / 6.0f);
    p = __builtin_fmaf(p, w, 1.0f / 5.0f);
    p = __builtin_fmaf(p, w, -1.0f / 4.0f);
    p = __builtin_fmaf(p, w, 1.0f / 3.0f);
    p = __builtin_fmaf(p, w, -0.5f);
    p = __builtin_fmaf(p, w, 1.0f);
    return p * w;
  }
  const float u = 1.0f + w;
  return log2_hw(u) * kLn2 * (w * rcp_hw(u - 1.0f));
}

// softplus(x) = ln(1 + e^x) = max(x, 0) + ln(1 + e^-|x|): no overflow for
// large x and no cancellation for very negative x.
__device__ __forceinline__ float softplus_f32(float x) {
  const float w = exp2_hw(-__builtin_fabsf(x) * kLog2e);
  return __builtin_fmaxf(x, 0.0f) + log1p_unit(w);
}

// silu(z) = z / (1 + e^-z).  For z -> -inf the reciprocal goes to 0 and the
// product to -0; no NaN for finite z.
__device__ __forceinline__ float silu_f32(float z) {
  return z * rcp_hw(1.0f + exp2_hw(-z * kLog2e));
}

// ---- element access for the two storage types ------------------------------
// float32 storage: float.  bfloat16 storage: uint16_t bit patterns.
template <typename T> struct Elem;

template <> struct Elem<float> {
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};

template <> struct Elem<uint16_t> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float load(const uint16_t* p) {
    return __uint_as_float(static_cast<uint32_t>(*p) << 16);
  }
  __device__ __forceinline__ static void store(uint16_t* p, float v) {
    const __bf16 h = static_cast<__bf16>(v);  // round to nearest even (v_cvt_pk_bf16_f32)
    *p = __builtin_bit_cast(uint16_t, h);
  }
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v.x = static_cast<__bf16>(lo);
  v.y = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// Load E consecutive elements starting at p into fp32 registers.  The caller
// guarantees all E are in range; `vec` says p is 16-byte aligned.
template <typename T, int E>
__device__ __forceinline__ void load_run(const T* __restrict__ p, bool vec, float (&out)[E]);

template <int E>
__device__ __forceinline__ void load_run(const float* __restrict__ p, bool vec, float (&out)[E]) {
  if (vec && (E % 4) == 0) {
#pragma unroll
    for (int i = 0; i < E / 4; ++i) {
      const float4 v = reinterpret_cast<const float4*>(p)[i];
      out[4 * i + 0] = v.x; out[4 * i + 1] = v.y; out[4 * i + 2] = v.z; out[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) out[i] = p[i];
  }
}

template <int E>
__device__ __forceinline__ void load_run(const uint16_t* __restrict__ p, bool vec, float (&out)[E]) {
  if (vec && (E % 8) == 0) {
#pragma unroll
    for (int i = 0; i < E / 8; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      out[8 * i + 0] = bf16_lo(v.x); out[8 * i + 1] = bf16_hi(v.x);
      out[8 * i + 2] = bf16_lo(v.y); out[8 * i + 3] = bf16_hi(v.y);
      out[8 * i + 4] = bf16_lo(v.z); out[8 * i + 5] = bf16_hi(v.z);
      out[8 * i + 6] = bf16_lo(v.w); out[8 * i + 7] = bf16_hi(v.w);
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) out[i] = Elem<uint16_t>::load(p + i);
  }
}

template <typename T, int E>
__device__ __forceinline__ void store_run(T* __restrict__ p, bool vec, const float (&v)[E]);

template <int E>
__device__ __forceinline__ void store_run(float* __restrict__ p, bool vec, const float (&v)[E]) {
  if (vec && (E % 4) == 0) {
#pragma unroll
    for (int i = 0; i < E / 4; ++i)
      reinterpret_cast<float4*>(p)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) p[i] = v[i];
  }
}

template <int E>
__device__ __forceinline__ void store_run(uint16_t* __restrict__ p, bool vec, const float (&v)[E]) {
  if (vec && (E % 8) == 0) {
#pragma unroll
    for (int i = 0; i < E / 8; ++i) {
      uint4 w;
      w.x = pack_bf16x2(v[8 * i + 0], v[8 * i + 1]);
      w.y = pack_bf16x2(v[8 * i + 2], v[8 * i + 3]);
      w.z = pack_bf16x2(v[8 * i + 4], v[8 * i + 5]);
      w.w = pack_bf16x2(v[8 * i + 6], v[8 * i + 7]);
      reinterpret_cast<uint4*>(p)[i] = w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) Elem<uint16_t>::store(p + i, v[i]);
  }
}

}  // namespace ssm
