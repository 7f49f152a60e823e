// state_update.hip -- one decode step of the selective scan for gfx950.
//
// Generation feeds one token at a time through the recurrence with a
// constant-size state per channel ("Exercises -- State-space models (Mamba,
// S4)", training vs generation: O(1) work and O(N) memory per token).  Per
// (b, d): Delta = softplus(delta + bias), then for each state
// h = exp(Delta*A)*h + Delta*B*u, and y = (C.h + D*u)*silu(z).
//
// The step is bound by reading and writing the fp32 state (N*8 bytes per
// channel against a few bytes of token input), so the layout is built for
// streaming it: NS = min(N, 4) states per lane (one 16-byte load and store),
// P = N/NS consecutive lanes per channel, so a wave reads and writes 1 KiB of
// state contiguously.  The P partial readouts are summed with lane shuffles
// in a fixed order.  The state's loads and stores are non-temporal: a
// channel's state is touched once per token, so keeping it in the caches
// only displaces other lines (measured on gfx950: 37.5 -> 33 us per step at
// batch 256, D 5120, N 16, against 35 and 37 us with only the loads or only
// the stores marked).
//
// Optional convolution prologue (the decode step of the causal depthwise
// conv1d + silu in front of the SSM): u = silu(cb + sum_k w[k] x[t-K+1+k])
// from the carried K-1 previous inputs and this token's x; the carried
// inputs are shifted in place to end with x.
#include "ssm_kernels.hpp"
#include "ssm_math.hpp"

namespace ssm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// A raw element of T as float.
__device__ __forceinline__ float raw_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ float raw_f32(float v) { return v; }

template <typename T, int N, int MODE, bool VEC, bool GATE>
__global__ __launch_bounds__(256) void state_update_kernel(
    float* __restrict__ state, const T* __restrict__ u, const T* __restrict__ delta,
    const float* __restrict__ A, const T* __restrict__ B, const T* __restrict__ C,
    const float* __restrict__ Dskip, const T* __restrict__ z, const float* __restrict__ bias,
    T* __restrict__ y, int b0, int dim, int softplus,
    float* __restrict__ conv_state, const float* __restrict__ conv_w,
    const float* __restrict__ conv_b, int conv_k) {
  // grid: (lanes of one batch row / 256, batch rows from b0); VEC: state, A,
  // B and C are aligned for the vector loads below
  constexpr bool ZOH = (MODE & kModeZoh) != 0;
  constexpr bool CONV = (MODE & kModeConv) != 0;
  constexpr int NS = N < 4 ? N : 4;
  constexpr int P = N / NS;
  const int idx = (int)blockIdx.x * 256 + (int)threadIdx.x;  // lane within the batch row
  // Whole channel groups of P lanes are either all in range or all out of
  // range (P divides 64 and idx ranges start at multiples of 64), so the
  // shuffles below only ever read lanes that are active.
  if (idx >= dim * P) return;
  const int b = b0 + (int)blockIdx.y;
  const int d = idx / P;
  const int part = idx % P;
  const int64_t row = (int64_t)b * dim + d;

  // ---- every load of the step, issued before any of them is used (one memory
  // round trip per thread); token values stay raw until then -------------------
  float h[NS], av[NS], bv[NS], cv[NS];
  float* sp = state + row * N + part * NS;
  const int64_t nb = (int64_t)b * N + part * NS;
  const float* ap = A + (int64_t)d * N + part * NS;
  uint32_t bw[2], cw[2];  // bf16 B, C of this lane's 4 states (VEC)
  if constexpr (NS == 4 && VEC) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sp));
    h[0] = v.x; h[1] = v.y; h[2] = v.z; h[3] = v.w;
    const float4 a4 = *reinterpret_cast<const float4*>(ap);
    av[0] = a4.x; av[1] = a4.y; av[2] = a4.z; av[3] = a4.w;
    if constexpr (sizeof(T) == 2) {
      const uint2 b2 = *reinterpret_cast<const uint2*>(B + nb);
      const uint2 c2 = *reinterpret_cast<const uint2*>(C + nb);
      bw[0] = b2.x; bw[1] = b2.y; cw[0] = c2.x; cw[1] = c2.y;
    } else {
      const float4 b4 = *reinterpret_cast<const float4*>(B + nb);
      const float4 c4 = *reinterpret_cast<const float4*>(C + nb);
      bv[0] = b4.x; bv[1] = b4.y; bv[2] = b4.z; bv[3] = b4.w;
      cv[0] = c4.x; cv[1] = c4.y; cv[2] = c4.z; cv[3] = c4.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      h[k] = __builtin_nontemporal_load(sp + k);
      av[k] = ap[k];
      bv[k] = raw_f32(B[nb + k]);
      cv[k] = raw_f32(C[nb + k]);
    }
  }
  const T u_raw = u[row];
  const T d_raw = delta[row];
  T z_raw = T(0);
  if constexpr (GATE) z_raw = z[row];
  const float bias_d = bias != nullptr ? bias[d] : 0.0f;
  const float D_d = Dskip != nullptr ? Dskip[d] : 0.0f;
  float prev[kMaxConvWidth - 1], taps[kMaxConvWidth], cbias = 0.0f;
  float* cs = nullptr;
  if constexpr (CONV) {
    cs = conv_state + row * (conv_k - 1);
#pragma unroll
    for (int j = 0; j < kMaxConvWidth - 1; ++j) prev[j] = j < conv_k - 1 ? cs[j] : 0.0f;
#pragma unroll
    for (int j = 0; j < kMaxConvWidth; ++j) taps[j] = j < conv_k ? conv_w[(int64_t)d * conv_k + j] : 0.0f;
    cbias = conv_b != nullptr ? conv_b[d] : 0.0f;
  }
  if constexpr (NS == 4 && VEC && sizeof(T) == 2) {
    bv[0] = bf16_lo(bw[0]); bv[1] = bf16_hi(bw[0]); bv[2] = bf16_lo(bw[1]); bv[3] = bf16_hi(bw[1]);
    cv[0] = bf16_lo(cw[0]); cv[1] = bf16_hi(cw[0]); cv[2] = bf16_lo(cw[1]); cv[3] = bf16_hi(cw[1]);
  }

  // ---- the step --------------------------------------------------------------
  float uv = raw_f32(u_raw);
  if constexpr (CONV) {
    // every lane of the channel forms u (a few FMAs); lane 0 shifts the
    // carried inputs.  The lanes of a channel are in one wave and lane 0
    // stores values its own loads returned, so the stores follow every
    // lane's loads of conv_state.
    const int K = conv_k;
    float sacc = cbias;
#pragma unroll
    for (int j = 0; j < kMaxConvWidth - 1; ++j)
      if (j < K - 1) sacc = __builtin_fmaf(taps[j], prev[j], sacc);
    sacc = __builtin_fmaf(taps[K - 1], uv, sacc);
    if (part == 0 && K > 1) {
#pragma unroll
      for (int j = 0; j < kMaxConvWidth - 2; ++j)
        if (j < K - 2) cs[j] = prev[j + 1];
      cs[K - 2] = uv;
    }
    uv = silu_f32(sacc);
  }
  const float x = raw_f32(d_raw) + bias_d;
  const float dt = softplus ? softplus_f32(x) : x;
  const float du = dt * uv;
  float acc = 0.0f;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const float x2 = dt * (av[k] * kLog2e);
    const float a = exp2_hw(x2);
    if constexpr (ZOH) {
      // zero-order hold: u*B * (exp(Delta A) - 1)/A
      h[k] = __builtin_fmaf(a, h[k], uv * bv[k] * zoh_coef(a, x2, dt, 1.0f / av[k]));
    } else {
      h[k] = __builtin_fmaf(a, h[k], du * bv[k]);
    }
    acc = __builtin_fmaf(cv[k], h[k], acc);
  }

  if constexpr (NS == 4 && VEC) {
    const f32x4 o = {h[0], h[1], h[2], h[3]};
    __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(sp));
  } else {
#pragma unroll
    for (int k = 0; k < NS; ++k) __builtin_nontemporal_store(h[k], sp + k);
  }

#pragma unroll
  for (int off = 1; off < P; off <<= 1) acc += __shfl_xor(acc, off);

  if (part == 0) {
    float yv = __builtin_fmaf(D_d, uv, acc);
    if constexpr (GATE) yv *= silu_f32(raw_f32(z_raw));
    Elem<T>::store(y + row, yv);
  }
}

template <typename T, int N, int MODE>
static hipError_t launch_n(const DecodeLaunch& a, hipStream_t stream) {
  constexpr int NS = N < 4 ? N : 4;
  constexpr int P = N / NS;
  const unsigned gx = (unsigned)(((int64_t)a.dim * P + 255) / 256);
  auto kernel = a.vec ? (a.z != nullptr ? state_update_kernel<T, N, MODE, true, true>
                                        : state_update_kernel<T, N, MODE, true, false>)
                      : (a.z != nullptr ? state_update_kernel<T, N, MODE, false, true>
                                        : state_update_kernel<T, N, MODE, false, false>);
  constexpr int kMaxRows = 65535;  // grid y per launch
  for (int b0 = 0; b0 < a.batch; b0 += kMaxRows) {
    const int nb = a.batch - b0 < kMaxRows ? a.batch - b0 : kMaxRows;
    kernel<<<dim3(gx, (unsigned)nb), 256, 0, stream>>>(
        a.state, static_cast<const T*>(a.u), static_cast<const T*>(a.delta), a.A,
        static_cast<const T*>(a.B), static_cast<const T*>(a.C), a.Dskip,
        static_cast<const T*>(a.z), a.bias, static_cast<T*>(a.y), b0, a.dim, a.softplus,
        a.conv_state, a.conv_w, a.conv_b, a.conv_k);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int MODE>
static hipError_t launch_t(const DecodeLaunch& a, hipStream_t stream) {
  switch (a.dstate) {
    case 1: return launch_n<T, 1, MODE>(a, stream);
    case 2: return launch_n<T, 2, MODE>(a, stream);
    case 4: return launch_n<T, 4, MODE>(a, stream);
    case 8: return launch_n<T, 8, MODE>(a, stream);
    case 16: return launch_n<T, 16, MODE>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t launch_mode(const DecodeLaunch& a, hipStream_t stream) {
  const int mode = (a.zoh ? kModeZoh : 0) | (a.conv_w != nullptr ? kModeConv : 0);
  switch (mode) {
    case 0: return launch_t<T, 0>(a, stream);
    case kModeZoh: return launch_t<T, kModeZoh>(a, stream);
    case kModeConv: return launch_t<T, kModeConv>(a, stream);
    default: return launch_t<T, kModeZoh | kModeConv>(a, stream);
  }
}

hipError_t launch_state_update(const DecodeLaunch& a, hipStream_t stream) {
  if (a.batch == 0 || a.dim == 0) return hipSuccess;
  if (a.conv_w != nullptr && (a.conv_k < 1 || a.conv_k > kMaxConvWidth)) return hipErrorInvalidValue;
  return a.dtype == Dtype::BF16 ? launch_mode<uint16_t>(a, stream) : launch_mode<float>(a, stream);
}

}  // namespace ssm
