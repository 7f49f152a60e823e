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

// v from the lane that the DPP control CTRL names (0 where it names none, or
// in rows that ROW_MASK leaves out).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_moved(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

// ln(1 + w) for w in [0, 1], without branches.  u = fl(1 + w) is rounded;
// c = w - (u - 1) is the rounding error exactly (u - 1 is exact), and
// ln(1 + w) = ln(u + c) = ln(u) + c/u + O(c^2).  Replacing c/u by c changes
// the result by c*(u - 1)/u, below half an ulp of ln(u) over the whole range,
// so ln(1 + w) = ln(u) + c to working precision.  When w is below half an
// ulp of 1, u = 1 and the result is c = w.  The hardware log2 keeps full
// relative precision for u just above 1.
__device__ __forceinline__ float log1p_unit(float w) {
  const float u = 1.0f + w;
  const float c = w - (u - 1.0f);
  return __builtin_fmaf(log2_hw(u), kLn2, c);
}

// softplus(x) = ln(1 + e^x) = max(x, 0) + ln(1 + e^-|x|): no overflow for
// large x and no cancellation for very negative x.  max(x, 0) is a signed
// integer max on the bits (one instruction; a float max would first quiet
// its input): a float with the sign bit clear is a non-negative integer.  A
// NaN x makes w, and so the result, NaN either way.
__device__ __forceinline__ float softplus_f32(float x) {
  const float w = exp2_hw(-__builtin_fabsf(x) * kLog2e);
  return __int_as_float(max(__float_as_int(x), 0)) + log1p_unit(w);
}

// Zero-order-hold input coefficient Bbar/B = (exp(Delta A) - 1)/A, given
// x2 = Delta*A*log2(e), a = exp2(x2), Delta and 1/A.  Where |Delta A| < 0.1
// the difference a - 1 would carry the rounding error of a magnified by
// 1/|Delta A|, so the Taylor series Delta*(1 + x/2 + x^2/6 + x^3/24),
// x = Delta A, is taken there (dropped terms below x^4/120 < 1e-6 relative);
// elsewhere (a - 1)/A, formed as one fma (relative error about 2^-23/0.1).
// A = 0 lands in the series and gives Delta, the limit.  Branch-free: both
// forms are computed and one is selected.
constexpr float kZohSeriesX2 = 0.1f * kLog2e;
__device__ __forceinline__ float zoh_coef(float a, float x2, float dt, float rA) {
  constexpr float k1 = kLn2 / 2.0f;
  constexpr float k2 = kLn2 * kLn2 / 6.0f;
  constexpr float k3 = kLn2 * kLn2 * kLn2 / 24.0f;
  const float p = __builtin_fmaf(x2, __builtin_fmaf(x2, __builtin_fmaf(x2, k3, k2), k1), 1.0f);
  const float series = dt * p;
  const float direct = __builtin_fmaf(a, rA, -rA);
  return __builtin_fabsf(x2) < kZohSeriesX2 ? series : direct;
}

// d/dA of the zero-order-hold coefficient (exp(Delta A) - 1)/A, for the
// backward pass: (x e^x - e^x + 1)/A^2 with x = Delta A, i.e. Delta^2 f(x)
// with f(x) = 1/2 + x/3 + x^2/8 + x^3/30 + x^4/144 + x^5/840 + ... (the
// series of (x e^x - e^x + 1)/x^2, term m-2 being (m-1)/m!).  The series is
// taken where abs(x) < 1/4 (truncation below 1e-7 relative; it is also the
// A = 0 limit Delta^2/2), the closed form elsewhere (its cancellation costs
// under 1e-6 relative there); both are computed and one is selected.
__device__ __forceinline__ float zoh_coef_dA(float a, float x2, float dt, float rA) {
  const float x = x2 * kLn2;
  const float f = __builtin_fmaf(
      x, __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 840.0f, 1.0f / 144.0f),
                                                                 1.0f / 30.0f),
                                          1.0f / 8.0f),
                        1.0f / 3.0f),
      0.5f);
  const float series = dt * dt * f;
  const float direct = __builtin_fmaf(x, a, 1.0f - a) * (rA * rA);
  return __builtin_fabsf(x) < 0.25f ? series : direct;
}

// The decay exp(A * SumDelta) of a whole segment, for composing segment
// aggregates: exp2(x), x = A*log2(e)*SumDelta, except that a result below
// the smallest normal float is raised to it while x is finite.  The decay
// over many steps can underflow where no single step's factor does; keeping
// it positive lets an infinite state stay infinite through the composition,
// as it does step by step (0 * inf would be NaN).  x = -inf (a step with
// Delta = inf, whose factor is exactly 0) still gives 0; NaN stays NaN.  On
// finite states the raise changes a result by at most 2^-126 times the
// state.
constexpr float kMinNormal = 1.17549435e-38f;
__device__ __forceinline__ float segment_decay(float x) {
  const float f = exp2_hw(x);
  return (f < kMinNormal && x > -__builtin_inff()) ? kMinNormal : f;
}

// silu(z) = z / (1 + e^-z).  For z -> -inf the reciprocal goes to 0 and the
// product to -0; no NaN for finite z.
__device__ __forceinline__ float silu_f32(float z) {
  return z * rcp_hw(1.0f + exp2_hw(-z * kLog2e));
}

// ---- element access for the two storage types ------------------------------
// float32 storage: float.  bfloat16 storage: uint16_t bit patterns.
// A compile-time bool as a value (selects an instantiation of a generic lambda).
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

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

// ---- buffer accesses ------------------------------------------------------------
// A buffer descriptor (base address and byte extent of a region, held in
// scalar registers) lets a lane address the region with a 32-bit offset that
// stays fixed while a scalar offset moves along the sequence: no per-lane
// 64-bit address arithmetic and two fewer VGPRs per stream.  Loads past the
// extent read 0 and stores past it are dropped.  Extents must be below 2^31
// bytes (the callers check it on the host).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
struct Buf {
  __amdgpu_buffer_rsrc_t r;
};
__device__ __forceinline__ Buf make_buf(const void* base, int64_t bytes) {
  return Buf{__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000)};
}

// W 32-bit words at voff + soff (W = 2: one 8-byte access; W = 4k: 16-byte ones).
template <int W>
__device__ __forceinline__ void buf_load_words(const Buf& b, uint32_t voff, uint32_t soff, uint32_t (&w)[W]) {
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(b.r, voff + 16 * i, soff, 0);
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  } else if constexpr (W == 2) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(b.r, voff, soff, 0);
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b32(b.r, voff + 4 * i, soff, 0);
  }
}

template <int W>
__device__ __forceinline__ void buf_store_words(const Buf& b, uint32_t voff, uint32_t soff, const uint32_t (&w)[W]) {
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      u32x4_t v;
      v.x = w[4 * i]; v.y = w[4 * i + 1]; v.z = w[4 * i + 2]; v.w = w[4 * i + 3];
      __builtin_amdgcn_raw_buffer_store_b128(v, b.r, voff + 16 * i, soff, 0);
    }
  } else if constexpr (W == 2) {
    u32x2_t v;
    v.x = w[0]; v.y = w[1];
    __builtin_amdgcn_raw_buffer_store_b64(v, b.r, voff, soff, 0);
  } else {
#pragma unroll
    for (int i = 0; i < W; ++i) __builtin_amdgcn_raw_buffer_store_b32(w[i], b.r, voff + 4 * i, soff, 0);
  }
}

// ---- vectorised runs of E consecutive elements ---------------------------------
// A run of E elements of T is W = E*sizeof(T)/4 32-bit words.  Callers pass
// pointers aligned to the run size (16 bytes when W is a multiple of 4).
template <int W>
__device__ __forceinline__ void load_words(const void* __restrict__ p, uint32_t (&w)[W]) {
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      w[4 * i + 0] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  } else if constexpr (W == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = reinterpret_cast<const uint32_t*>(p)[i];
  }
}

template <int W>
__device__ __forceinline__ void store_words(void* __restrict__ p, const uint32_t (&w)[W]) {
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int i = 0; i < W / 4; ++i)
      reinterpret_cast<uint4*>(p)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  } else if constexpr (W == 2) {
    *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
  } else {
#pragma unroll
    for (int i = 0; i < W; ++i) reinterpret_cast<uint32_t*>(p)[i] = w[i];
  }
}

template <typename T, int E>
__device__ __forceinline__ void words_to_floats(const uint32_t (&w)[E * sizeof(T) / 4], float (&f)[E]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) f[i] = __uint_as_float(w[i]);
  }
}

// Pack E floats into the words of T storage (bf16: round to nearest even).
template <typename T, int E>
__device__ __forceinline__ void pack_floats(const float (&f)[E], uint32_t (&w)[E * sizeof(T) / 4]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < E / 2; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) w[i] = __float_as_uint(f[i]);
  }
}

// Store E floats as T (bf16: round to nearest even) with vector stores.
template <typename T, int E>
__device__ __forceinline__ void store_floats(T* __restrict__ p, const float (&f)[E]) {
  constexpr int W = E * (int)sizeof(T) / 4;
  uint32_t w[W];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = __float_as_uint(f[i]);
  }
  store_words<W>(p, w);
}

}  // namespace ssm
