// scan_fwd.hip -- the fused selective-scan forward pass for gfx950.
//
// What it computes is stated in include/ssm.h: per channel (b, d) and state
// n, Delta = softplus(delta + bias), Abar = exp(Delta*A) (zero-order hold,
// "Mamba" paper review, "SSM"), input term Delta*B*u (the Euler form named
// in the "Paper: Mamba" course module), h = Abar*h + Delta*B*u, and the
// readout y = (C.h + D*u)*silu(z) after each update ("Exercises --
// State-space models (Mamba, S4)", recurrent view).
//
// Design (channel-parallel, one fused pass over HBM):
//  * A workgroup owns 64 consecutive channels of one batch row and G state
//    groups; wave g holds NS = N/G states of each of its 64 channels in
//    VGPRs (lane = channel).  The state never touches HBM.
//  * The sequence is walked in tiles of TL steps.  Per tile, all threads
//    load u, delta (and z) with coalesced 16-byte loads along L, compute
//    Delta = softplus(delta + bias) and Delta*u once per element, and stage
//    them transposed in LDS (one float2 per (t, channel)).
//  * Each wave then runs the TL steps of the recurrence for its states.
//    B[b,n,t] and C[b,n,t] are the same for every lane of a wave (shared by
//    all channels), so they are scalar loads, not VGPR traffic.  Per
//    (element, state) the loop is one v_exp_f32 and four fp32 VALU ops.
//  * The G partial readouts per (t, channel) are summed through LDS in a
//    fixed order, D*u and the silu gate applied, and y stored with coalesced
//    16-byte stores.
//  * Long sequences with too few channels to fill the GPU are split into
//    segments.  The affine steps compose associatively ("NN LAB" Mamba page,
//    "The Associative Property of Linear Recurrence"): a first launch runs
//    every segment but the last from a zero state (segment 0 from h0) and
//    records its end state and the sum of its Delta; the main launch then
//    starts segment s from the composition of those aggregates,
//    h_in(s) = exp(A * SumDelta(s-1)) * h_in(s-1) + h_end(s-1),
//    which is exact up to rounding, and writes y once.
#include "ssm_kernels.hpp"
#include "ssm_math.hpp"

namespace ssm {

struct ScanSizes {
  int batch, dim;
  int64_t seqlen;
  int64_t seglen;
  int nseg;          // segments of the sequence
  int nseg_launch;   // segments covered by this launch
  int ncg;           // 64-channel groups per batch row
  int softplus;
  int vec;
};

template <typename T, int NS, int G, int TL, bool AGG>
__global__ __launch_bounds__(64 * G) void scan_kernel(
    const T* __restrict__ u, const T* __restrict__ delta, const float* __restrict__ A,
    const T* __restrict__ B, const T* __restrict__ C, const float* __restrict__ Dskip,
    const T* __restrict__ z, const float* __restrict__ bias, const float* __restrict__ h0,
    T* __restrict__ y, float* __restrict__ last_state, float* __restrict__ ws_hend,
    float* __restrict__ ws_sumdt, const ScanSizes p) {
  constexpr int N = NS * G;
  constexpr int E = TL / G;  // elements per thread in the load / store phases
  static_assert(TL % G == 0, "tile must split evenly over the state groups");

  __shared__ float2 s_ddu[TL][64];                            // (Delta, Delta*u)
  __shared__ float s_y[AGG ? 1 : G][AGG ? 1 : TL][64];        // partial readouts

  // ---- block -> (batch row, channel group, segment) --------------------------
  // Consecutive block ids go to different XCDs; regroup so that the blocks an
  // XCD runs share batch rows (and hence B and C in that XCD's L2).
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int seg = bid % p.nseg_launch;
  const int rest = bid / p.nseg_launch;
  const int cg = rest % p.ncg;
  const int b = rest / p.ncg;

  const int tid = threadIdx.x;
  const int g = __builtin_amdgcn_readfirstlane(tid >> 6);  // state group (wave-uniform)
  const int lane = tid & 63;                                // channel in the group
  const int64_t L = p.seqlen;
  const int d = cg * 64 + lane;
  const bool dvalid = d < p.dim;
  const int64_t row = (int64_t)b * p.dim + d;

  const int64_t seg_begin = (int64_t)seg * p.seglen;
  const int64_t seg_end = seg_begin + p.seglen < L ? seg_begin + p.seglen : L;

  // ---- per-lane parameters and initial state ---------------------------------
  float A2[NS], h[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const int n = g * NS + k;
    A2[k] = dvalid ? A[(int64_t)d * N + n] * kLog2e : 0.0f;
    h[k] = 0.0f;
    if (seg == 0 && h0 != nullptr && dvalid) h[k] = h0[row * N + n];
  }
  if (!AGG && seg > 0 && dvalid) {
    // carry-in: compose the aggregates of segments 0 .. seg-1 in order
    const int64_t plane = (int64_t)p.batch * p.dim;
#pragma unroll
    for (int k = 0; k < NS; ++k) h[k] = ws_hend[row * N + g * NS + k];
    for (int j = 1; j < seg; ++j) {
      const float sdt = ws_sumdt[j * plane + row];
#pragma unroll
      for (int k = 0; k < NS; ++k)
        h[k] = __builtin_fmaf(exp2_hw(sdt * A2[k]), h[k], ws_hend[(j * plane + row) * N + g * NS + k]);
    }
  }

  // ---- load-phase role: thread -> (channel cc, run of E steps) ---------------
  const int cc = tid / G;
  const int chunk = tid % G;
  const int dcc = cg * 64 + cc;
  const bool ccvalid = dcc < p.dim;
  const int64_t rowcc = (int64_t)b * p.dim + dcc;
  const float bias_cc = (bias != nullptr && ccvalid) ? bias[dcc] : 0.0f;
  const float D_cc = (Dskip != nullptr && ccvalid) ? Dskip[dcc] : 0.0f;
  const bool has_z = (z != nullptr);

  const T* Bw = B + ((int64_t)b * N + g * NS) * L;  // wave-uniform
  const T* Cw = C + ((int64_t)b * N + g * NS) * L;

  double sumdt = 0.0;

  for (int64_t t0 = seg_begin; t0 < seg_end; t0 += TL) {
    const int tvalid = (int)((seg_end - t0) < TL ? (seg_end - t0) : TL);
    const int r0 = chunk * E;                  // first step of this thread's run
    const int rn = tvalid - r0;                // steps of the run in range
    const bool full = rn >= E;

    // ---- load u, delta (z), form Delta and Delta*u, stage in LDS -------------
    float uu[E], dd[E], zz[E];
    if (ccvalid && full) {
      const int64_t off = rowcc * L + t0 + r0;
      load_run<E>(u + off, p.vec != 0, uu);
      load_run<E>(delta + off, p.vec != 0, dd);
      if (!AGG && has_z) load_run<E>(z + off, p.vec != 0, zz);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool ok = ccvalid && e < rn;
        const int64_t off = rowcc * L + t0 + r0 + e;
        uu[e] = ok ? Elem<T>::load(u + off) : 0.0f;
        dd[e] = ok ? Elem<T>::load(delta + off) : 0.0f;
        zz[e] = (ok && !AGG && has_z) ? Elem<T>::load(z + off) : 0.0f;
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float x = dd[e] + bias_cc;
      float dt = p.softplus ? softplus_f32(x) : x;
      if (!(ccvalid && e < rn)) dt = 0.0f;
      s_ddu[r0 + e][cc] = make_float2(dt, dt * uu[e]);
    }
    __syncthreads();

    // ---- the recurrence: TL steps x NS states per lane -------------------------
    const T* Bt = Bw + t0;
    const T* Ct = Cw + t0;
    if (tvalid == TL) {
#pragma unroll 4
      for (int t = 0; t < TL; ++t) {
        const float2 v = s_ddu[t][lane];
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < NS; ++k) {
          const float bv = Elem<T>::load(Bt + (int64_t)k * L + t);
          const float cv = Elem<T>::load(Ct + (int64_t)k * L + t);
          const float a = exp2_hw(v.x * A2[k]);
          h[k] = __builtin_fmaf(a, h[k], v.y * bv);
          acc = __builtin_fmaf(cv, h[k], acc);
        }
        if (!AGG) s_y[AGG ? 0 : g][AGG ? 0 : t][lane] = acc;
        if (AGG && g == 0) sumdt += (double)v.x;
      }
    } else {
      for (int t = 0; t < tvalid; ++t) {
        const float2 v = s_ddu[t][lane];
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < NS; ++k) {
          const float bv = Elem<T>::load(Bt + (int64_t)k * L + t);
          const float cv = Elem<T>::load(Ct + (int64_t)k * L + t);
          const float a = exp2_hw(v.x * A2[k]);
          h[k] = __builtin_fmaf(a, h[k], v.y * bv);
          acc = __builtin_fmaf(cv, h[k], acc);
        }
        if (!AGG) s_y[AGG ? 0 : g][AGG ? 0 : t][lane] = acc;
        if (AGG && g == 0) sumdt += (double)v.x;
      }
    }
    __syncthreads();

    // ---- readout: sum the G partials, D-skip, gate, store y --------------------
    if (!AGG) {
      float yv[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float s = 0.0f;
#pragma unroll
        for (int gg = 0; gg < G; ++gg) s += s_y[AGG ? 0 : gg][AGG ? 0 : r0 + e][cc];
        s = __builtin_fmaf(D_cc, uu[e], s);
        if (has_z) s *= silu_f32(zz[e]);
        yv[e] = s;
      }
      if (ccvalid) {
        const int64_t off = rowcc * L + t0 + r0;
        if (full) {
          store_run<E>(y + off, p.vec != 0, yv);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e)
            if (e < rn) Elem<T>::store(y + off + e, yv[e]);
        }
      }
    }
    // The next tile's LDS writes (s_ddu) are not read by this readout, and its
    // s_y writes come after the next barrier, so no third barrier is needed.
  }

  // ---- segment results ---------------------------------------------------------
  if (!dvalid) return;
  if (AGG) {
    const int64_t plane = (int64_t)p.batch * p.dim;
#pragma unroll
    for (int k = 0; k < NS; ++k) ws_hend[(seg * plane + row) * N + g * NS + k] = h[k];
    if (g == 0) ws_sumdt[seg * plane + row] = (float)sumdt;
  } else if (last_state != nullptr && seg == p.nseg - 1) {
#pragma unroll
    for (int k = 0; k < NS; ++k) last_state[row * N + g * NS + k] = h[k];
  }
}

template <typename T, int NS, int G>
static hipError_t launch_typed(const ScanLaunch& a, hipStream_t stream) {
  constexpr int TL = kScanTile;
  ScanSizes s;
  s.batch = a.batch;
  s.dim = a.dim;
  s.seqlen = a.seqlen;
  s.seglen = a.seglen;
  s.nseg = a.nseg;
  s.ncg = (a.dim + 63) / 64;
  s.softplus = a.softplus;
  s.vec = a.vec;
  const T* u = static_cast<const T*>(a.u);
  const T* dl = static_cast<const T*>(a.delta);
  const T* B = static_cast<const T*>(a.B);
  const T* C = static_cast<const T*>(a.C);
  const T* z = static_cast<const T*>(a.z);
  T* y = static_cast<T*>(a.y);
  const int64_t base = (int64_t)a.batch * s.ncg;
  if (a.nseg > 1) {
    s.nseg_launch = a.nseg - 1;
    const unsigned grid = (unsigned)(base * s.nseg_launch);
    scan_kernel<T, NS, G, TL, true><<<grid, 64 * G, 0, stream>>>(
        u, dl, a.A, B, C, a.Dskip, z, a.bias, a.h0, y, a.last_state, a.ws_hend, a.ws_sumdt, s);
  }
  s.nseg_launch = a.nseg;
  const unsigned grid = (unsigned)(base * s.nseg_launch);
  scan_kernel<T, NS, G, TL, false><<<grid, 64 * G, 0, stream>>>(
      u, dl, a.A, B, C, a.Dskip, z, a.bias, a.h0, y, a.last_state, a.ws_hend, a.ws_sumdt, s);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_by_state(const ScanLaunch& a, hipStream_t stream) {
  switch (a.dstate) {
    case 1: return launch_typed<T, 1, 1>(a, stream);
    case 2: return launch_typed<T, 2, 1>(a, stream);
    case 4: return launch_typed<T, 4, 1>(a, stream);
    case 8: return launch_typed<T, 4, 2>(a, stream);
    case 16: return launch_typed<T, 4, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scan_fwd(const ScanLaunch& a, hipStream_t stream) {
  if (a.batch == 0 || a.dim == 0 || a.seqlen == 0) return hipSuccess;
  return a.dtype == Dtype::BF16 ? launch_by_state<uint16_t>(a, stream)
                                : launch_by_state<float>(a, stream);
}

__global__ void fill_state_kernel(float* __restrict__ dst, const float* __restrict__ src, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src != nullptr ? src[i] : 0.0f;
}

hipError_t launch_fill_state(float* dst, const float* src, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  fill_state_kernel<<<grid, 256, 0, stream>>>(dst, src, n);
  return hipGetLastError();
}

}  // namespace ssm
