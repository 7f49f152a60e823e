// valu_rate.hip -- issue rate of the VALU instruction mixes the scan kernels
// are made of, on one gfx950 GPU.  A standalone program (no library, no
// torch): each kernel runs independent chains of one mix in every lane, with
// 1 to 8 waves per SIMD, and the rate is printed as wave-instructions per
// SIMD per nanosecond.  One fp32 VALU instruction of a wave takes 4 clocks on
// a 16-lane SIMD, so the plain-fma rate times 4 is the sustained clock in GHz.
//
//   fma      8 chains of fma: 8 VALU instructions per iteration
//   exp      8 chains of x = exp2(x) * c: 8 exp + 8 multiplies per iteration
//   mul      8 chains of multiplies by a scalar (SGPR) or per-lane (VGPR)
//            factor
//   scan     the forward scan's recurrence, 4 states and 2 steps per
//            iteration: per (step, state) a multiply (Delta A log2 e),
//            exp2, a multiply (Delta u B), the state fma and the readout fma
//            (B, C, A per state): 46 VALU instructions per iteration in
//            the compiled loop, 8 of them exp (40 for the 8 (step, state)
//            updates, the rest forming the step values); A per lane as in
//            the kernel, B and C as scalar operands or held in VGPRs
//   scan, no input product
//            the same recurrence with Delta u added to the state unscaled:
//            the rate the mix would reach if the multiply by B cost nothing
//   scan, input product on the matrix core
//            per step one v_mfma_f32_4x4x1_16b_f32 forms the 4 states'
//            Delta u * B at once (the 16 blocks of 4x4 outer products: lane
//            l supplies B[l % 4] and its own Delta u, and its 4 result
//            registers hold Delta u * B[r], r = 0..3)
//
// Build: hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops
//        -mllvm -amdgpu-mfma-vgpr-form valu_rate.hip -o valu_rate
// (the last option lets the matrix instruction write VGPRs directly, where
// the default would route its result through AGPRs and VALU moves)
#include <hip/hip_runtime.h>
#include <cstdio>

namespace {

constexpr int kIters = 4096;

__global__ __launch_bounds__(256) void fma_kernel(float* out, float a, float b) {
  float x[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) x[c] = threadIdx.x * 1e-3f + c;
  for (int i = 0; i < kIters; ++i) {
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = __builtin_fmaf(x[c], a, b);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += x[c];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void exp_kernel(float* out, float a, float) {
  float x[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) x[c] = threadIdx.x * 1e-6f + c * 1e-3f;
  for (int i = 0; i < kIters; ++i) {
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = __builtin_amdgcn_exp2f(x[c]) * a;
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += x[c];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// plain multiplies by a scalar operand (SGPR) or by a per-lane one (VGPR)
template <bool VGPR>
__global__ __launch_bounds__(256) void mul_kernel(float* out, float a, float) {
  float x[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) x[c] = threadIdx.x * 1e-3f + c;
  float m = a;
  if constexpr (VGPR) asm volatile("" : "+v"(m));  // keep the factor in a VGPR
  for (int i = 0; i < kIters; ++i) {
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = x[c] * m;
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += x[c];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

struct ScanParams {
  float A2[4], B[4], C[4];
};

// VGPR_BC: B and C held in VGPRs instead of read as scalar operands
template <bool VGPR_BC>
__global__ __launch_bounds__(256) void scan_kernel(float* out, ScanParams p, float) {
  float h[4] = {0.0f, 0.0f, 0.0f, 0.0f}, acc = 0.0f;
  float A2[4], B[4], C[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    A2[k] = p.A2[k];
    B[k] = p.B[k];
    C[k] = p.C[k];
    asm volatile("" : "+v"(A2[k]));  // per-lane in the scan kernel: a VGPR
    if constexpr (VGPR_BC) {
      asm volatile("" : "+v"(B[k]));
      asm volatile("" : "+v"(C[k]));
    }
  }
  float dt = 0.01f + threadIdx.x * 1e-6f, du = 0.5f;
  for (int i = 0; i < kIters; ++i) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float d = dt + s * 1e-4f, q = du - s * 1e-4f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a = __builtin_amdgcn_exp2f(d * A2[k]);
        h[k] = __builtin_fmaf(a, h[k], q * B[k]);
        acc = __builtin_fmaf(C[k], h[k], acc);
      }
    }
    dt = dt * 0.9999f + 1e-6f;
    du = du * 0.9999f;
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc + h[0] + h[1] + h[2] + h[3];
}

typedef float float4v __attribute__((ext_vector_type(4)));

// The recurrence of scan_kernel with B as scalar operands, but the input
// product Delta u * B either left out (MFMA false: the state takes Delta u
// itself) or formed on the matrix core (MFMA true)
template <bool MFMA>
__global__ __launch_bounds__(256) void scan_input_kernel(float* out, ScanParams p, float) {
  float h[4] = {0.0f, 0.0f, 0.0f, 0.0f}, acc = 0.0f;
  float A2[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    A2[k] = p.A2[k];
    asm volatile("" : "+v"(A2[k]));
  }
  const int q4 = threadIdx.x & 3;
  float bvec = q4 == 0 ? p.B[0] : q4 == 1 ? p.B[1] : q4 == 2 ? p.B[2] : p.B[3];
  asm volatile("" : "+v"(bvec));
  float dt = 0.01f + threadIdx.x * 1e-6f, du = 0.5f;
  for (int i = 0; i < kIters; ++i) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float d = dt + s * 1e-4f, q = du - s * 1e-4f;
      float4v qv = {q, q, q, q};
      if constexpr (MFMA) {
        const float4v zero = {0.0f, 0.0f, 0.0f, 0.0f};
        qv = __builtin_amdgcn_mfma_f32_4x4x1f32(bvec, q, zero, 0, 0, 0);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a = __builtin_amdgcn_exp2f(d * A2[k]);
        h[k] = __builtin_fmaf(a, h[k], qv[k]);
        acc = __builtin_fmaf(p.C[k], h[k], acc);
      }
    }
    dt = dt * 0.9999f + 1e-6f;
    du = du * 0.9999f;
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc + h[0] + h[1] + h[2] + h[3];
}

template <typename F, typename P>
float time_ms(F f, int blocks, float* out, P p, float b) {
  hipEvent_t e0, e1;
  hipEventCreate(&e0);
  hipEventCreate(&e1);
  hipLaunchKernelGGL(f, dim3(blocks), dim3(256), 0, 0, out, p, b);
  hipEventRecord(e0, 0);
  for (int r = 0; r < 5; ++r) hipLaunchKernelGGL(f, dim3(blocks), dim3(256), 0, 0, out, p, b);
  hipEventRecord(e1, 0);
  hipEventSynchronize(e1);
  float ms = 0.0f;
  hipEventElapsedTime(&ms, e0, e1);
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  return ms / 5.0f;
}

}  // namespace

int main() {
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess || ncu <= 0) return 1;
  float* out = nullptr;
  const int max_blocks = ncu * 8;  // 8 workgroups of 4 waves per CU: 8 waves per SIMD
  if (hipMalloc(&out, (size_t)max_blocks * 256 * sizeof(float)) != hipSuccess) return 1;
  const ScanParams sp = {{-1.4427f, -2.885f, -4.328f, -5.770f}, {0.3f, -0.2f, 0.1f, 0.4f}, {0.5f, 0.25f, -0.3f, 0.2f}};
  const int waves_per_simd[] = {1, 2, 3, 5, 8};
  printf("{\"cus\": %d, \"iterations\": %d}\n", ncu, kIters);
  for (int w : waves_per_simd) {
    const int blocks = ncu * w;
    const double wave_iters_per_simd = (double)blocks * 4 * kIters / (ncu * 4.0);
    const float t_fma = time_ms(fma_kernel, blocks, out, 0.999f, 1e-3f);
    const float t_exp = time_ms(exp_kernel, blocks, out, 0.999f, 0.0f);
    const float t_scan = time_ms(scan_kernel<false>, blocks, out, sp, 0.0f);
    const float t_scan_v = time_ms(scan_kernel<true>, blocks, out, sp, 0.0f);
    const float t_mul_s = time_ms(mul_kernel<false>, blocks, out, 0.999f, 0.0f);
    const float t_mul_v = time_ms(mul_kernel<true>, blocks, out, 0.999f, 0.0f);
    const float t_noq = time_ms(scan_input_kernel<false>, blocks, out, sp, 0.0f);
    const float t_mfma = time_ms(scan_input_kernel<true>, blocks, out, sp, 0.0f);
    const double r_fma = wave_iters_per_simd * 8 / (t_fma * 1e6);
    const double r_exp = wave_iters_per_simd * 16 / (t_exp * 1e6);
    const double r_scan = wave_iters_per_simd * 46 / (t_scan * 1e6);
    printf("{\"waves_per_simd\": %d, \"fma\": %.4f, \"mul_sgpr\": %.4f, \"mul_vgpr\": %.4f, \"exp_mul\": %.4f, "
           "\"scan\": %.4f, \"scan_element_states_per_simd_ns\": %.3f, \"scan_bc_vgpr_element_states_per_simd_ns\": %.3f, "
           "\"scan_no_input_product_element_states_per_simd_ns\": %.3f, "
           "\"scan_mfma_input_product_element_states_per_simd_ns\": %.3f, \"clock_ghz_from_fma\": %.3f}\n",
           w, r_fma, wave_iters_per_simd * 8 / (t_mul_s * 1e6), wave_iters_per_simd * 8 / (t_mul_v * 1e6), r_exp, r_scan,
           wave_iters_per_simd * 8 * 64 / (t_scan * 1e6), wave_iters_per_simd * 8 * 64 / (t_scan_v * 1e6),
           wave_iters_per_simd * 8 * 64 / (t_noq * 1e6), wave_iters_per_simd * 8 * 64 / (t_mfma * 1e6), 4.0 * r_fma);
  }
  hipFree(out);
  return 0;
}
