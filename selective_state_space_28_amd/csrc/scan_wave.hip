// scan_wave.hip -- the forward scan for long sequences with few channels,
// parallel over time inside each wave.
//
// It computes what scan_fwd.hip computes (include/ssm.h states it): per
// channel and state Delta = softplus(delta + bias), Abar = exp(Delta A), the
// input term Delta*B*u (Euler) or (Abar - 1)/A*B*u (zero-order hold),
// h = Abar h + input term and y = (C.h + D u) silu(z) after each update.
//
// The channel-parallel kernel gives each lane a channel; with few channels
// and long sequences (batch 1, D 2048, L 65536) it must split every sequence
// into segments and run it twice (segment aggregates, then the main pass).
// Here a wave holds one channel and 4 of its 16 states, and its 64 lanes own
// 64 consecutive chunks of kWaveChunk steps: a block of 64 * kWaveChunk steps
// at a time.  Per block:
//  1. staging: the workgroup's threads form Delta and the input factor
//     (Delta u, or u under zero-order hold) of its kWaveChannels channels, and
//     put the block's B and C in LDS, laid out so that every lane reads its
//     own steps without bank conflicts;
//  2. local pass: each lane runs its chunk from a zero state, keeping each
//     step's Abar and input term in registers, and forms the chunk's affine
//     map h -> P h + hl with P = exp(A * the chunk's Delta sum);
//  3. the maps are composed over the lanes by an inclusive prefix (DPP row
//     shifts, then row broadcasts) with the associative operator of the
//     NN LAB "Mamba" page ("The Associative Property of Linear Recurrence"):
//     (P2, h2) after (P1, h1) is (P2 P1, P2 h1 + h2).  The state entering the
//     block is folded into lane 0 first, so lane j ends with the state after
//     its chunk, and the lane before it holds the state entering it;
//  4. fix-up: each lane reruns its chunk from that state with the kept
//     factors (no exponentials), forming its 4 states' part of C.h per step;
//  5. readout: the 4 state groups' parts are summed through LDS in a fixed
//     order, D u added, the gate applied and y stored.
// The state after lane 63's chunk enters the next block.  Steps past the end
// of the sequence are identity steps (Delta = 0, no input).
#include "ssm_kernels.hpp"
#include "ssm_math.hpp"

namespace ssm {

namespace {

constexpr int kWaveChunk = 8;                    // steps per lane and block
constexpr int kWaveBlock = 64 * kWaveChunk;      // steps per block
constexpr int kWaveChannels = 4;                 // channels per workgroup
constexpr int kWaveN = 16;                       // states (4 groups of 4)
constexpr int kWaveNS = 4;                       // states per wave

struct WaveSizes {
  int batch, dim;
  int64_t seqlen;
  int softplus;
  int vec_io;  // u, delta, z, y: 16-byte aligned rows of 16-byte multiples (pairs of elements as one access)
  int vec_bc;  // B, C: the same (a chunk's steps of one state as whole 16-byte accesses)
};

// One round of the prefix over the wave: lanes that the DPP control CTRL
// (with ROW_MASK) gives a source compose their map after the source lane's;
// the others read the identity (h 0, P 1) and keep theirs.  A composed decay
// that underflows is raised to the smallest normal float, as a segment's
// decay is (segment_decay), so that an infinite state stays infinite through
// the composition, as it does step by step.  (A range holding a step with
// Delta = inf, whose decay is exactly 0, is also raised; its own state is
// then infinite or NaN already.)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void compose_round(float (&P)[kWaveNS], float (&h)[kWaveNS]) {
#pragma unroll
  for (int k = 0; k < kWaveNS; ++k) {
    const float hf = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(h[k]), CTRL, ROW_MASK, 0xf, true));
    const float pf =
        __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(P[k]), CTRL, ROW_MASK, 0xf, false));
    h[k] = __builtin_fmaf(P[k], hf, h[k]);
    P[k] = __builtin_fmaxf(P[k] * pf, kMinNormal);
  }
}

// Raw bits of one element of T (zero when !ok).
template <typename T>
__device__ __forceinline__ uint32_t raw_elem(const T* __restrict__ p, bool ok);
template <>
__device__ __forceinline__ uint32_t raw_elem<float>(const float* __restrict__ p, bool ok) {
  return ok ? __float_as_uint(*p) : 0u;
}
template <>
__device__ __forceinline__ uint32_t raw_elem<uint16_t>(const uint16_t* __restrict__ p, bool ok) {
  return ok ? static_cast<uint32_t>(*p) : 0u;
}

// E consecutive elements p[0 .. E-1] as the words of T (those from `valid` on
// read as zero): one vector access when `vec`, else element loads.
template <typename T, int E>
__device__ __forceinline__ void load_elems(const T* __restrict__ p, bool vec, int64_t valid,
                                           uint32_t (&w)[E * sizeof(T) / 4]) {
  constexpr int W = E * (int)sizeof(T) / 4;
  if (vec) {
    load_words<W>(p, w);
  } else if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < W; ++i)
      w[i] = raw_elem<T>(p + 2 * i, 2 * i < valid) | (raw_elem<T>(p + 2 * i + 1, 2 * i + 1 < valid) << 16);
  } else {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = raw_elem<T>(p + i, i < valid);
  }
}

}  // namespace

template <typename T, bool ZOH>
__global__ __launch_bounds__(64 * 4 * kWaveChannels) void scan_wave_kernel(
    const T* __restrict__ u, const T* __restrict__ delta, const float* __restrict__ A,
    const T* __restrict__ B, const T* __restrict__ C, const float* __restrict__ Dskip,
    const T* __restrict__ z, const float* __restrict__ bias, const float* __restrict__ h0,
    T* __restrict__ y, float* __restrict__ last_state, const WaveSizes p) {
  constexpr int TC = kWaveChunk, N = kWaveN, NS = kWaveNS, G = N / NS;
  // (Delta, input factor) of channel c at step j*TC + i of the block
  __shared__ float2 s_d[kWaveChannels][TC][64];
  // B (0) and C (1) of states 4g .. 4g+3 at step j*TC + i: lane j reads 16
  // consecutive bytes, so a wave's reads of one i are conflict-free
  __shared__ float4 s_bc[2][TC][G][64];
  // each state group's part of C.h of channel c at step j*TC + i
  __shared__ float s_y[kWaveChannels][G][TC][64];

  const int tid = threadIdx.x;
  const int ncg = (p.dim + kWaveChannels - 1) / kWaveChannels;
  const int b = blockIdx.x / ncg;
  const int cgrp = blockIdx.x % ncg;
  const int64_t L = p.seqlen;

  // ---- recurrence role: wave -> (channel c, state group g), lane j -> chunk j --
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = w / G, g = w % G;
  const int j = tid & 63;
  const int d = cgrp * kWaveChannels + c;
  const bool dvalid = d < p.dim;
  const int64_t row = (int64_t)b * p.dim + (dvalid ? d : 0);
  float A2[NS], rA[NS], H[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const int n = g * NS + k;
    const float av = dvalid ? A[(int64_t)d * N + n] : -1.0f;
    A2[k] = dvalid ? av * kLog2e : 0.0f;
    rA[k] = 1.0f / av;  // zero-order-hold input term only
    H[k] = (dvalid && h0 != nullptr) ? h0[row * N + n] : 0.0f;
  }

  // ---- element role: thread -> (channel cs, steps e0, e0 + 1 of a block) -------
  const int cs = tid >> 8;
  const int e0 = (tid & 255) * 2;
  const int dcs = cgrp * kWaveChannels + cs;
  const bool csvalid = dcs < p.dim;
  const int64_t rcs = ((int64_t)b * p.dim + (csvalid ? dcs : 0)) * L;
  const float bias_c = (bias != nullptr && csvalid) ? bias[dcs] : 0.0f;
  const float D_c = (Dskip != nullptr && csvalid) ? Dskip[dcs] : 0.0f;
  const bool has_z = z != nullptr;

  // ---- record role: thread -> (state rn, the TC steps of chunk tid & 63) ------
  const int rn = tid >> 6;
  const int rj = tid & 63;
  const T* const Brow = B + ((int64_t)b * N + rn) * L + rj * TC;
  const T* const Crow = C + ((int64_t)b * N + rn) * L + rj * TC;

  // the next block's inputs, loaded while the current block runs, as raw
  // words of T (bf16 pairs share a word)
  constexpr int WE = 2 * (int)sizeof(T) / 4;   // a thread's 2 elements
  constexpr int WB = TC * (int)sizeof(T) / 4;  // a chunk's TC steps of one state
  uint32_t wu[WE], wd[WE], wz[WE], wb[WB], wc[WB];
  auto fetch = [&](int64_t tb) {
    const bool full = tb + kWaveBlock <= L;
    const int64_t ve = csvalid ? L - (tb + e0) : 0;
    load_elems<T, 2>(u + rcs + tb + e0, full && csvalid && p.vec_io, ve, wu);
    load_elems<T, 2>(delta + rcs + tb + e0, full && csvalid && p.vec_io, ve, wd);
    if (has_z) load_elems<T, 2>(z + rcs + tb + e0, full && csvalid && p.vec_io, ve, wz);
    const int64_t vb = L - (tb + rj * TC);
    load_elems<T, TC>(Brow + tb, full && p.vec_bc, vb, wb);
    load_elems<T, TC>(Crow + tb, full && p.vec_bc, vb, wc);
  };

  const int64_t nblk = (L + kWaveBlock - 1) / kWaveBlock;
  fetch(0);
  for (int64_t blk = 0; blk < nblk; ++blk) {
    const int64_t tb = blk * kWaveBlock;

    // ---- 1. staging ---------------------------------------------------------------
    uint32_t eu[WE], ez[WE];  // this block's u and z, for the readout
    {
      float fu[2], fd[2];
      words_to_floats<T, 2>(wu, fu);
      words_to_floats<T, 2>(wd, fd);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int s = e0 + m;
        const bool ok = csvalid && tb + s < L;
        const float x = fd[m] + bias_c;
        const float dt = ok ? (p.softplus ? softplus_f32(x) : x) : 0.0f;  // past the end: identity steps
        const float xin = ok ? (ZOH ? fu[m] : dt * fu[m]) : 0.0f;
        s_d[cs][s % TC][s / TC] = make_float2(dt, xin);
      }
#pragma unroll
      for (int i = 0; i < WE; ++i) {
        eu[i] = wu[i];
        ez[i] = has_z ? wz[i] : 0u;
      }
      float fb[TC], fc[TC];
      words_to_floats<T, TC>(wb, fb);
      words_to_floats<T, TC>(wc, fc);
#pragma unroll
      for (int m = 0; m < TC; ++m) {
        reinterpret_cast<float*>(&s_bc[0][m][rn / NS][rj])[rn % NS] = fb[m];
        reinterpret_cast<float*>(&s_bc[1][m][rn / NS][rj])[rn % NS] = fc[m];
      }
    }
    if (blk + 1 < nblk) fetch(tb + kWaveBlock);
    __syncthreads();

    // ---- 2. local pass of chunk j from a zero state ------------------------------------
    float ah[TC][NS], qh[TC][NS], hl[NS], S = 0.0f;
#pragma unroll
    for (int k = 0; k < NS; ++k) hl[k] = 0.0f;
#pragma unroll
    for (int i = 0; i < TC; ++i) {
      const float2 v = s_d[c][i][j];
      const float4 bq = s_bc[0][i][g][j];
      const float bb[NS] = {bq.x, bq.y, bq.z, bq.w};
      S += v.x;
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const float x2 = v.x * A2[k];
        const float a = exp2_hw(x2);
        const float q = ZOH ? zoh_coef(a, x2, v.x, rA[k]) * (v.y * bb[k]) : v.y * bb[k];
        ah[i][k] = a;
        qh[i][k] = q;
        hl[k] = __builtin_fmaf(a, hl[k], q);
      }
    }

    // ---- 3. compose the chunks' maps over the wave -------------------------------------
    float P[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      P[k] = segment_decay(S * A2[k]);
      if (j == 0) hl[k] = __builtin_fmaf(P[k], H[k], hl[k]);  // the state entering the block
    }
    compose_round<0x111, 0xf>(P, hl);  // row_shr:1
    compose_round<0x112, 0xf>(P, hl);  // row_shr:2
    compose_round<0x114, 0xf>(P, hl);  // row_shr:4
    compose_round<0x118, 0xf>(P, hl);  // row_shr:8
    compose_round<0x142, 0xa>(P, hl);  // row_bcast:15 into rows 1 and 3
    compose_round<0x143, 0xc>(P, hl);  // row_bcast:31 into rows 2 and 3
    float hs[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      // the state entering chunk j: lane j-1's (wave_shr:1), lane 0 the block's
      hs[k] = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(H[k]), __float_as_int(hl[k]), 0x138, 0xf, 0xf, false));
      H[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hl[k]), 63));
    }

    // ---- 4. fix-up: the chunk again from its true state ---------------------------------
#pragma unroll
    for (int i = 0; i < TC; ++i) {
      const float4 cq = s_bc[1][i][g][j];
      const float cc[NS] = {cq.x, cq.y, cq.z, cq.w};
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        hs[k] = __builtin_fmaf(ah[i][k], hs[k], qh[i][k]);
        acc = __builtin_fmaf(cc[k], hs[k], acc);
      }
      s_y[c][g][i][j] = acc;
    }
    __syncthreads();

    // ---- 5. readout: sum the state groups' parts, D-skip, gate, store y ---------------
    float yv[2], fu[2], fz[2];
    words_to_floats<T, 2>(eu, fu);
    words_to_floats<T, 2>(ez, fz);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int s = e0 + m;
      float sum = s_y[cs][0][s % TC][s / TC];
#pragma unroll
      for (int gg = 1; gg < G; ++gg) sum += s_y[cs][gg][s % TC][s / TC];
      sum = __builtin_fmaf(D_c, fu[m], sum);
      if (has_z) sum *= silu_f32(fz[m]);
      yv[m] = sum;
    }
    if (csvalid) {
      const int64_t t = tb + e0;
      if (p.vec_io && t + 1 < L) {
        store_floats<T, 2>(y + rcs + t, yv);
      } else {
#pragma unroll
        for (int m = 0; m < 2; ++m)
          if (t + m < L) Elem<T>::store(y + rcs + t + m, yv[m]);
      }
    }
    // The next block's staging writes s_d and s_bc, which only steps 2 and 4
    // read (before the barrier above); s_y is written again only after the
    // next block's first barrier.
  }

  if (dvalid && last_state != nullptr && j == 0) {
#pragma unroll
    for (int k = 0; k < NS; ++k) last_state[row * N + g * NS + k] = H[k];
  }
}

template <typename T, bool ZOH>
static hipError_t launch_wave_typed(const ScanLaunch& a, hipStream_t stream) {
  WaveSizes s;
  s.batch = a.batch;
  s.dim = a.dim;
  s.seqlen = a.seqlen;
  s.softplus = a.softplus;
  s.vec_io = a.vec;
  s.vec_bc = a.vec_bc;
  const int64_t grid = (int64_t)a.batch * ((a.dim + kWaveChannels - 1) / kWaveChannels);
  scan_wave_kernel<T, ZOH><<<(unsigned)grid, 64 * 4 * kWaveChannels, 0, stream>>>(
      static_cast<const T*>(a.u), static_cast<const T*>(a.delta), a.A, static_cast<const T*>(a.B),
      static_cast<const T*>(a.C), a.Dskip, static_cast<const T*>(a.z), a.bias, a.h0, static_cast<T*>(a.y),
      a.last_state, s);
  return hipGetLastError();
}

hipError_t launch_scan_wave(const ScanLaunch& a, hipStream_t stream) {
  if (a.batch == 0 || a.dim == 0 || a.seqlen == 0) return hipSuccess;
  if (a.dstate != kWaveN || a.conv_w != nullptr || a.ws_ckpt != nullptr) return hipErrorInvalidValue;
  if (a.dtype == Dtype::BF16)
    return a.zoh ? launch_wave_typed<uint16_t, true>(a, stream) : launch_wave_typed<uint16_t, false>(a, stream);
  return a.zoh ? launch_wave_typed<float, true>(a, stream) : launch_wave_typed<float, false>(a, stream);
}

}  // namespace ssm
