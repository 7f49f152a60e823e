// scan_bwd.hip -- backward pass of the selective scan for gfx950.
//
// Gradients of a loss L through y = scan(u, delta, A, B, C, D, z, bias, h0)
// given dy = dL/dy (and optionally dL/dlast_state), by recomputation: the
// "Mamba" paper review ("Optimization") notes that the intermediate states
// needed for backpropagation are cheaper to recompute from the inputs than
// to store (B*L*D*N elements).  Here:
//
//  1. The forward kernel's checkpoint pass (scan_fwd.hip) stores the state
//     entering every 16-step tile: 1/16 of the states, (batch, tile, N, dim).
//  2. The adjoint lambda_t = dL/dh_t obeys its own linear recurrence
//     backwards in time, lambda_t = ds_t C_t + Abar_{t+1} lambda_{t+1}
//     (ds_t = dL/d(pre-gate output)), independent of h.  When the sequence
//     is split into segments, bwd_agg_kernel runs each segment but the first
//     from a zero carry; the carry entering segment s from the right is then
//     the composition mu_s = exp(A SumDelta_{s+1}) mu_{s+1} + Q_{s+1} -- the
//     associative affine step of the NN LAB "Mamba" page, run in reverse.
//  3. bwd_kernel walks each segment's tiles from last to first: it
//     recomputes the tile's 16 states from the checkpoint into registers,
//     keeping each step's Abar (and the zero-order-hold coefficient) beside
//     them so the sweep need not form them again, then sweeps the steps in
//     reverse, carrying lambda per state and forming every gradient term.  dB and dC are sums over channels: each
//     wave sums its terms over its 64 channels in registers with lane
//     exchanges (permlane swaps and DPP), a few steps at a time, and writes
//     them as per-channel-group partials.  dA, dD and the bias gradient are
//     per-workgroup partials.  A tile takes three workgroup barriers.
//  4. Small kernels sum the partials in a fixed order, so results are
//     deterministic.
//
// Per (element, state) the gradient terms are (Euler input term):
//   lambda = ds C + carry;  carry' = Abar lambda
//   dA    += lambda h_{t-1} Abar Delta
//   dDelta += lambda (h_{t-1} Abar A + B u)
//   du    += lambda Delta B;   dB += lambda Delta u;   dC += ds h_t
// With the zero-order-hold term Bbar = (Abar - 1)/A in place of Delta
// (dBbar/dDelta = Abar, dBbar/dA from zoh_coef_dA):
//   dA    += lambda (h_{t-1} Abar Delta + dBbar/dA B u)
//   dDelta += lambda (h_{t-1} Abar A + Abar B u)
//   du    += lambda Bbar B;    dB += lambda Bbar u
// and per element du += ds D, dD += ds u, d(delta) = dDelta softplus'(x),
// dz = dy (C.h + D u) silu'(z), ds = dy silu(z).
#include "ssm_kernels.hpp"
#include "ssm_math.hpp"

namespace ssm {

struct BwdSizes {
  int batch, dim;
  int64_t seqlen, seglen;
  int nseg;
  int ncg;
  int softplus;
  int vec;
};

__device__ __forceinline__ float sigmoid_f32(float x) { return rcp_hw(1.0f + exp2_hw(-x * kLog2e)); }

// Sums of 16 values per lane over the 64 lanes of a wave: lane l returns the
// total of value (l >> 2) & 15.  Each round pairs every lane with a partner;
// the pair splits its values in halves, each lane keeps one half and adds the
// partner's copy of it: lanes l, l^32 (v_permlane32_swap), l, l^16
// (v_permlane16_swap), l, l^8 (DPP row_ror:8, a select for the half kept)
// and l, l^7 (DPP row_half_mirror).  Two quad permutes then add l^2 and l^1.
// The order of the additions is fixed, so the sums are deterministic.
__device__ __forceinline__ float wave_sum16(const float (&v)[16], int lane) {
  float r[8], q[4], h2[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[j]), __float_as_uint(v[j + 8]), false, false);
    r[j] = __uint_as_float(s[0]) + __uint_as_float(s[1]);  // value j + 8 (l >> 5 & 1)
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(r[j]), __float_as_uint(r[j + 4]), false, false);
    q[j] = __uint_as_float(s[0]) + __uint_as_float(s[1]);  // + 4 (l >> 4 & 1)
  }
  const bool b3 = (lane & 8) != 0, b2 = (lane & 4) != 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float keep = b3 ? q[j + 2] : q[j], send = b3 ? q[j] : q[j + 2];
    h2[j] = keep + dpp_moved<0x128, 0xf>(send);  // + 2 (l >> 3 & 1)
  }
  const float keep = b2 ? h2[1] : h2[0], send = b2 ? h2[0] : h2[1];
  float w = keep + dpp_moved<0x141, 0xf>(send);  // + (l >> 2 & 1)
  w += dpp_moved<0x4e, 0xf>(w);                  // quad_perm [2,3,0,1]
  w += dpp_moved<0xb1, 0xf>(w);                  // quad_perm [1,0,3,2]
  return w;
}

// Value q of a B, C record (scalar loads; see scan_fwd.hip for the layout).
template <typename T>
__device__ __forceinline__ float bwd_rec(const T* __restrict__ p, int q);
template <>
__device__ __forceinline__ float bwd_rec<float>(const float* __restrict__ p, int q) { return p[q]; }
template <>
__device__ __forceinline__ float bwd_rec<uint16_t>(const uint16_t* __restrict__ p, int q) {
  const uint32_t w = reinterpret_cast<const uint32_t*>(p)[q >> 1];
  return (q & 1) ? bf16_hi(w) : bf16_lo(w);
}

// E consecutive elements of one row starting at off: a vector load when the
// run is whole and aligned, else element loads (zeros past `valid`).
template <typename T, int E>
__device__ __forceinline__ void load_run(const T* __restrict__ base, int64_t off, bool vec_ok, int valid,
                                         float (&f)[E]) {
  constexpr int W = E * (int)sizeof(T) / 4;
  if (vec_ok) {
    uint32_t w[W];
    load_words<W>(base + off, w);
    words_to_floats<T, E>(w, f);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = e < valid ? Elem<T>::load(base + off + e) : 0.0f;
  }
}

// Per-element gradients are written once and never read back here: their
// stores are non-temporal, so they do not displace from L2 the input lines
// that the earlier tiles of the same lines still need.
template <typename T, int E>
__device__ __forceinline__ void store_run(T* __restrict__ base, int64_t off, bool vec_ok, int valid,
                                          const float (&f)[E]) {
  if (vec_ok) {
    constexpr int W = E * (int)sizeof(T) / 4;
    uint32_t w[W];
    pack_floats<T, E>(f, w);
    if constexpr (W == 2) {
      __builtin_nontemporal_store(((uint64_t)w[1] << 32) | w[0], reinterpret_cast<uint64_t*>(base + off));
    } else {
#pragma unroll
      for (int i = 0; i < W; ++i) __builtin_nontemporal_store(w[i], reinterpret_cast<uint32_t*>(base + off) + i);
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (e < valid) Elem<T>::store(base + off + e, f[e]);
  }
}

// A whole run of E elements through a buffer descriptor, non-temporal (the
// slc bit of the cache policy: nt on this architecture).
template <typename T, int E>
__device__ __forceinline__ void buf_store_run_nt(const Buf& bb, uint32_t voff, uint32_t soff, const float (&f)[E]) {
  constexpr int W = E * (int)sizeof(T) / 4;
  uint32_t w[W];
  pack_floats<T, E>(f, w);
  if constexpr (W == 1) {
    __builtin_amdgcn_raw_buffer_store_b32(w[0], bb.r, voff, soff, 2);
  } else if constexpr (W == 2) {
    u32x2_t v;
    v.x = w[0]; v.y = w[1];
    __builtin_amdgcn_raw_buffer_store_b64(v, bb.r, voff, soff, 2);
  } else {
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      u32x4_t v;
      v.x = w[4 * i]; v.y = w[4 * i + 1]; v.z = w[4 * i + 2]; v.w = w[4 * i + 3];
      __builtin_amdgcn_raw_buffer_store_b128(v, bb.r, voff + 16 * i, soff, 2);
    }
  }
}

// ---- 2. reverse aggregates of segments 1 .. nseg-1 ------------------------------
template <typename T, int NS, int G, int TL>
__global__ __launch_bounds__(64 * G) void bwd_agg_kernel(
    const T* __restrict__ delta, const float* __restrict__ A, const T* __restrict__ bc,
    const T* __restrict__ z, const float* __restrict__ bias, const T* __restrict__ dy,
    float* __restrict__ lagg, float* __restrict__ lsum, const BwdSizes p) {
  constexpr int N = NS * G;
  constexpr int E = TL / G;
  constexpr int LDW = 65;
  constexpr int R = 2 * NS;
  __shared__ float2 s_v[TL][LDW];  // (Delta, ds)

  const int nlaunch = p.nseg - 1;
  const int seg = 1 + (int)(blockIdx.x % nlaunch);
  const int rest = (int)(blockIdx.x / nlaunch);
  const int cg = rest % p.ncg;
  const int b = rest / p.ncg;
  const int tid = threadIdx.x;
  const int g = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int64_t L = p.seqlen;
  const int d = cg * 64 + lane;
  const bool dvalid = d < p.dim;
  const int64_t row = (int64_t)b * p.dim + d;
  const int64_t seg_begin = (int64_t)seg * p.seglen;
  const int64_t seg_end = seg_begin + p.seglen < L ? seg_begin + p.seglen : L;

  float A2[NS], carry[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    A2[k] = dvalid ? A[(int64_t)d * N + g * NS + k] * kLog2e : 0.0f;
    carry[k] = 0.0f;
  }
  const int cc = tid / G;
  const int r0 = (tid % G) * E;
  const int dcc = cg * 64 + cc;
  const bool ccvalid = dcc < p.dim;
  const int64_t rowcc = (int64_t)b * p.dim + (ccvalid ? dcc : 0);
  const float bias_cc = (bias != nullptr && ccvalid) ? bias[dcc] : 0.0f;
  const T* bcw = bc + ((int64_t)b * G + g) * L * R;
  double sumdt = 0.0;

  for (int64_t t0 = ((seg_end - 1) / TL) * TL; t0 >= seg_begin; t0 -= TL) {
    const int tvalid = (int)((seg_end - t0) < TL ? (seg_end - t0) : TL);
    {
      const int valid = ccvalid ? (tvalid - r0 < 0 ? 0 : (tvalid - r0 > E ? E : tvalid - r0)) : 0;
      const bool vec_ok = p.vec && valid == E;
      const int64_t off = rowcc * L + t0 + r0;
      float dd[E], gg[E], zz[E];
      load_run<T, E>(delta, off, vec_ok, valid, dd);
      load_run<T, E>(dy, off, vec_ok, valid, gg);
      if (z != nullptr) load_run<T, E>(z, off, vec_ok, valid, zz);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float x = dd[e] + bias_cc;
        const float dt = p.softplus ? softplus_f32(x) : x;
        const float ds = z != nullptr ? gg[e] * silu_f32(zz[e]) : gg[e];
        s_v[r0 + e][cc] = make_float2(dt, e < valid ? ds : 0.0f);
      }
    }
    __syncthreads();
    const T* bct = bcw + t0 * R;
    for (int t = tvalid - 1; t >= 0; --t) {
      const float2 v = s_v[t][lane];
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const float lam = __builtin_fmaf(v.y, bwd_rec<T>(bct + t * R, NS + k), carry[k]);
        carry[k] = exp2_hw(v.x * A2[k]) * lam;
      }
      if (g == 0) sumdt += (double)v.x;
    }
    __syncthreads();
  }
  if (!dvalid) return;
  const int64_t plane = (int64_t)p.batch * p.dim;
#pragma unroll
  for (int k = 0; k < NS; ++k) lagg[((int64_t)(seg - 1) * plane + row) * N + g * NS + k] = carry[k];
  if (g == 0) lsum[(int64_t)(seg - 1) * plane + row] = (float)sumdt;
}

// ---- 3. the main backward sweep --------------------------------------------------
// Wave g holds NS states of each of the workgroup's 64 channels.  The B, C
// records are packed in groups of RNS states (the forward pass's layout);
// RNS may be larger than NS.  The zero-order-hold instantiation carries more
// live values per (element, state), so it runs with half the states per wave
// and twice the waves where RNS >= 2 (NS = RNS / 2, one workgroup per CU).
template <typename T, int NS, int G, int TL, bool ZOH, int RNS>
__global__ __launch_bounds__(64 * G, ZOH ? 1 : 2) void bwd_kernel(
    const T* __restrict__ u, const T* __restrict__ delta, const float* __restrict__ A,
    const T* __restrict__ bc, const float* __restrict__ Dskip, const T* __restrict__ z,
    const float* __restrict__ bias, const T* __restrict__ dy, const float* __restrict__ dlast,
    const float* __restrict__ ckpt, const float* __restrict__ lagg, const float* __restrict__ lsum,
    T* __restrict__ du, T* __restrict__ ddelta, T* __restrict__ dz, float* __restrict__ dh0,
    float* __restrict__ part_bc, float* __restrict__ part_a, float* __restrict__ part_d,
    float* __restrict__ part_bias, const BwdSizes p) {
  constexpr int N = NS * G;
  constexpr int E = TL / G;                   // elements per thread, element role
  constexpr int TRS = 8 / NS;                 // steps per dB/dC wave sum (16 terms a lane)
  constexpr int LDW = 65;                     // padded row, float/float2/float4 arrays
  constexpr int R = 2 * RNS;                  // values of a record: RNS B values, then RNS C values
  constexpr int RG = N / RNS;                 // record groups
  static_assert(NS * TRS == 8 && TL % TRS == 0, "dB/dC sums take 16 terms a lane");
  static_assert(RNS % NS == 0 && N % RNS == 0 && TL % G == 0, "state groups");

  __shared__ float4 s_in[TL][LDW];            // (Delta, Delta*u, ds, u) per (step, channel)
  __shared__ float s_y[G][TL][LDW];           // readout partials of each wave
  // per wave and step, the sums over this wave's states: Euler (sum lambda B,
  // the Abar part of dDelta); ZOH (sum lambda Bbar B, u sum lambda Abar B plus
  // the Abar part of dDelta)
  __shared__ float2 s_p[G][TL][LDW];
  // this tile's B, C records of every record group as floats, [group][t][q]:
  // loaded a tile ahead with the other inputs, read by each wave as broadcasts
  __shared__ __align__(16) float s_rec[RG][TL][R];

  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int seg = bid % p.nseg;
  const int rest = bid / p.nseg;
  const int cg = rest % p.ncg;
  const int b = rest / p.ncg;

  const int tid = threadIdx.x;
  const int g = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int64_t L = p.seqlen;
  const int d = cg * 64 + lane;
  const bool dvalid = d < p.dim;
  const int64_t row = (int64_t)b * p.dim + d;
  const int64_t seg_begin = (int64_t)seg * p.seglen;
  const int64_t seg_end = seg_begin + p.seglen < L ? seg_begin + p.seglen : L;
  const int64_t ntiles = (L + TL - 1) / TL;
  // this wave's states n = g NS + k sit in record group n / RNS at position
  // n % RNS: B of state k at rec_w[t R + k], C at rec_w[t R + RNS + k]
  const float* const rec_w = &s_rec[0][0][0] + (g * NS / RNS) * (TL * R) + (g * NS) % RNS;
  const int64_t plane = (int64_t)p.batch * p.dim;

  // ---- recurrence role: parameters and the carry entering the segment's end --
  float A2[NS], rA[NS], carry[NS], dA[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const int n = g * NS + k;
    const float av = dvalid ? A[(int64_t)d * N + n] : 0.0f;
    A2[k] = av * kLog2e;
    rA[k] = 1.0f / av;  // used by the zero-order-hold forms only, where A = 0 takes the series
    carry[k] = (dvalid && dlast != nullptr) ? dlast[row * N + n] : 0.0f;
    dA[k] = 0.0f;
  }
  if (dvalid) {
    for (int j = p.nseg - 1; j > seg; --j) {
      const float sdt = lsum[(int64_t)(j - 1) * plane + row];
#pragma unroll
      for (int k = 0; k < NS; ++k)
        carry[k] = __builtin_fmaf(segment_decay(sdt * A2[k]), carry[k],
                                  lagg[((int64_t)(j - 1) * plane + row) * N + g * NS + k]);
    }
  }

  // ---- element role: thread -> (channel cc, run of E steps) --------------------
  const int cc = tid / G;
  const int chunk = tid % G;
  const int r0 = chunk * E;
  const int dcc = cg * 64 + cc;
  const bool ccvalid = dcc < p.dim;
  const int64_t rowcc = (int64_t)b * p.dim + (ccvalid ? dcc : 0);
  const float bias_cc = (bias != nullptr && ccvalid) ? bias[dcc] : 0.0f;
  const float D_cc = (Dskip != nullptr && ccvalid) ? Dskip[dcc] : 0.0f;
  const bool has_z = z != nullptr;
  // whole tiles address the workgroup's 64 rows through buffer descriptors:
  // a lane's 32-bit offset is fixed, the tile's step offset is a scalar
  const int64_t grow = (int64_t)b * p.dim + (int64_t)cg * 64;
  const int64_t gbytes = p.vec ? (int64_t)min(64, p.dim - cg * 64) * L * (int64_t)sizeof(T) : 0;
  const Buf b_u = make_buf(u + grow * L, gbytes);
  const Buf b_dl = make_buf(delta + grow * L, gbytes);
  const Buf b_g = make_buf(dy + grow * L, gbytes);
  const Buf b_z = make_buf(has_z ? z + grow * L : u, has_z ? gbytes : 0);
  const Buf b_du = make_buf(du + grow * L, gbytes);
  const Buf b_dd = make_buf(ddelta + grow * L, gbytes);
  const Buf b_dz = make_buf(has_z ? dz + grow * L : du, has_z ? gbytes : 0);
  const uint32_t voff = p.vec ? (uint32_t)(((int64_t)cc * L + r0) * (int64_t)sizeof(T)) : 0u;
  float accD = 0.0f, accBias = 0.0f;

  float hist[TL][NS];
  // Abar of each step and state, and the zero-order-hold coefficient, kept
  // from the recompute for the sweep where the registers allow (few state
  // groups give long element runs, whose registers leave no room: there the
  // sweep forms Abar again)
  constexpr bool KEEP = ZOH || G >= 4;
  float ahist[KEEP ? TL : 1][KEEP ? NS : 1];
  float chist[ZOH ? TL : 1][ZOH ? NS : 1];
  // where this lane writes its wave sums of the dB, dC terms (lanes 4o write
  // term o of a group; see the reverse sweep)
  const int so = lane >> 2;
  float* const pbc = part_bc + ((((int64_t)b * p.ncg + cg) * 2 + (so >> 3)) * N + g * NS + (so / TRS) % NS) * L +
                     so % TRS;

  // A whole tile (FULL: all TL steps in the segment, rows 16-byte aligned) takes
  // its element runs and its checkpoint from registers loaded while the
  // previous tile ran, and has no per-step guards; a ragged tile loads its own.
  constexpr int W = E * (int)sizeof(T) / 4;
  // one tile ahead when a thread's runs are at most 16 bytes (few states give
  // long runs; those tiles load their own inputs, still without guards)
  constexpr bool PF = W <= 4;
  uint32_t pu[W], pd[W], pg[W], pz[W];  // the next whole tile's runs, raw
  float pck[NS];                          // and the state entering it
  // record staging: pair q of the tile's G * TL * R record values (group q /
  // (TL R / 2), values 2 (q % (TL R / 2)) and the next), one pair per thread
  constexpr int NPAIR = RG * TL * R / 2;
  constexpr int PW = (int)sizeof(T) / 2;  // words of a pair
  static_assert(NPAIR <= 64 * G, "one record pair per thread at most");
  const bool rec_thread = tid < NPAIR;
  const int rec_g = tid / (TL * R / 2), rec_e = 2 * (tid % (TL * R / 2));
  const T* bc_rec = bc + ((int64_t)b * RG + (rec_thread ? rec_g : 0)) * L * R + rec_e;
  uint32_t prec[PW];
  auto load_rec = [&](int64_t t0, bool guard, uint32_t (&w)[PW]) {
    const int tt = rec_e / R;  // the step of this pair (both values share it: R is even)
    if (!rec_thread || (guard && t0 + tt >= L)) {
#pragma unroll
      for (int i = 0; i < PW; ++i) w[i] = 0u;
    } else {
      load_words<PW>(bc_rec + t0 * R, w);
    }
  };
  auto prefetch = [&](int64_t t0) {
    const uint32_t so = (uint32_t)t0 * (uint32_t)sizeof(T);
    buf_load_words<W>(b_u, voff, so, pu);
    buf_load_words<W>(b_dl, voff, so, pd);
    buf_load_words<W>(b_g, voff, so, pg);
    if (has_z) buf_load_words<W>(b_z, voff, so, pz);
    load_rec(t0, false, prec);
    // (non-temporal: each checkpoint is read once, and kept out of L2 it
    // leaves room for the input lines that the next tiles read again)
#pragma unroll
    for (int k = 0; k < NS; ++k)
      pck[k] = dvalid ? __builtin_nontemporal_load(&ckpt[(((int64_t)b * ntiles + t0 / TL) * N + g * NS + k) * p.dim + d]) : 0.0f;
  };

  auto tile = [&](auto full_c, int64_t t0, int64_t next) {
    constexpr bool FULL = decltype(full_c)::value;
    const int tvalid = FULL ? TL : (int)((seg_end - t0) < TL ? (seg_end - t0) : TL);
    const int valid = FULL ? (ccvalid ? E : 0)
                           : (ccvalid ? (tvalid - r0 < 0 ? 0 : (tvalid - r0 > E ? E : tvalid - r0)) : 0);
    const bool vec_ok = FULL || (p.vec && valid == E);
    const int64_t eoff = rowcc * L + t0 + r0;
    if constexpr (FULL && !PF) prefetch(t0);

    // ---- stage: Delta, Delta*u, ds, u -------------------------------------------
    float e_u[E], e_ds[E], e_sg[E], e_gz[E], e_dt[E];
    {
      float uu[E], dd[E], gg[E], zz[E];
      if constexpr (FULL) {
        words_to_floats<T, E>(pu, uu);
        words_to_floats<T, E>(pd, dd);
        words_to_floats<T, E>(pg, gg);
        if (has_z) words_to_floats<T, E>(pz, zz);
      } else {
        load_run<T, E>(u, eoff, vec_ok, valid, uu);
        load_run<T, E>(delta, eoff, vec_ok, valid, dd);
        load_run<T, E>(dy, eoff, vec_ok, valid, gg);
        if (has_z) load_run<T, E>(z, eoff, vec_ok, valid, zz);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float x = dd[e] + bias_cc;
        const float dt = p.softplus ? softplus_f32(x) : x;
        float ds = gg[e], gz = 0.0f;
        if (has_z) {
          const float sz = sigmoid_f32(zz[e]);
          ds = gg[e] * (zz[e] * sz);
          gz = gg[e] * sz * __builtin_fmaf(zz[e], 1.0f - sz, 1.0f);
        }
        if (e >= valid) ds = 0.0f;
        e_u[e] = uu[e];
        e_ds[e] = ds;
        e_sg[e] = p.softplus ? sigmoid_f32(x) : 1.0f;
        e_gz[e] = gz;
        e_dt[e] = dt;
        s_in[r0 + e][cc] = make_float4(dt, dt * uu[e], ds, uu[e]);
      }
    }
    {
      uint32_t rw[PW];
      if constexpr (FULL) {
#pragma unroll
        for (int i = 0; i < PW; ++i) rw[i] = prec[i];
      } else {
        load_rec(t0, true, rw);
      }
      if (rec_thread) {
        float f[2];
        words_to_floats<T, 2>(rw, f);
        *reinterpret_cast<float2*>(&s_rec[rec_g][rec_e / R][rec_e % R]) = make_float2(f[0], f[1]);
      }
    }
    __syncthreads();

    // ---- recompute the tile's states from its checkpoint ------------------------
    float hp0[NS];
    if constexpr (FULL) {
#pragma unroll
      for (int k = 0; k < NS; ++k) hp0[k] = pck[k];
      if constexpr (PF) prefetch(next);  // the registers of this tile are consumed
    } else {
#pragma unroll
      for (int k = 0; k < NS; ++k)
        hp0[k] = dvalid ? ckpt[(((int64_t)b * ntiles + t0 / TL) * N + g * NS + k) * p.dim + d] : 0.0f;
    }
    {
      float h[NS];
#pragma unroll
      for (int k = 0; k < NS; ++k) h[k] = hp0[k];
#pragma unroll
      for (int t = 0; t < TL; ++t) {
        if (FULL || t < tvalid) {
          const float4 v = s_in[t][lane];
          float acc = 0.0f;
#pragma unroll
          for (int k = 0; k < NS; ++k) {
            const float x2 = v.x * A2[k];
            const float a = exp2_hw(x2);
            if constexpr (ZOH)
            {
              const float coef = zoh_coef(a, x2, v.x, rA[k]);
              chist[ZOH ? t : 0][ZOH ? k : 0] = coef;
              h[k] = __builtin_fmaf(a, h[k], coef * (v.w * rec_w[t * R + k]));
            }
            else
              h[k] = __builtin_fmaf(a, h[k], v.y * rec_w[t * R + k]);
            hist[t][k] = h[k];
            if constexpr (KEEP) ahist[t][k] = a;
            acc = __builtin_fmaf(rec_w[t * R + RNS + k], h[k], acc);
          }
          s_y[g][t][lane] = acc;
        }
      }
    }
    __syncthreads();

    // ---- dz = dy (C.h + D u) silu'(z) ---------------------------------------------
    if (has_z) {
      float zo[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float s = 0.0f;
        if (e < valid) {
#pragma unroll
          for (int gg = 0; gg < G; ++gg) s += s_y[gg][r0 + e][cc];
        }
        zo[e] = e_gz[e] * __builtin_fmaf(D_cc, e_u[e], s);
      }
      if constexpr (FULL) buf_store_run_nt<T, E>(b_dz, voff, (uint32_t)t0 * (uint32_t)sizeof(T), zo);
      else if (valid > 0) store_run<T, E>(dz, eoff, vec_ok, valid, zo);
    }

    // ---- reverse sweep, in groups of TRS steps ----------------------------------
    // A group's 16 dB and dC terms per lane (TRS steps x NS states) are summed
    // over the wave's 64 channels in registers; the per-step sums over the
    // wave's states, for du and d(delta), go to LDS for the whole tile.
#pragma unroll
    for (int grp = TL / TRS - 1; grp >= 0; --grp) {
      if (!FULL && grp * TRS >= tvalid) continue;  // uniform: a ragged last tile
      float terms[16];  // [w * 8 + k * TRS + i]: w = 0 the dB term, 1 the dC term
#pragma unroll
      for (int q = 0; q < 16; ++q) terms[q] = 0.0f;
#pragma unroll
      for (int i = TRS - 1; i >= 0; --i) {
        const int t = grp * TRS + i;
        float lb = 0.0f, la = 0.0f, dd = 0.0f;
        if (FULL || t < tvalid) {
          const float4 v = s_in[t][lane];
#pragma unroll
          for (int k = 0; k < NS; ++k) {
            const float x2 = v.x * A2[k];
            const float a = KEEP ? ahist[KEEP ? t : 0][KEEP ? k : 0] : exp2_hw(x2);
            const float lam = __builtin_fmaf(v.z, rec_w[t * R + RNS + k], carry[k]);
            const float hp = t > 0 ? hist[t > 0 ? t - 1 : 0][k] : hp0[k];
            const float cn = a * lam;  // the carry into step t - 1
            const float gh = cn * hp;
            dd = __builtin_fmaf(gh, A2[k], dd);
            if constexpr (ZOH) {
              // input term Bbar B u with Bbar = (Abar - 1)/A: dBbar/dDelta = Abar
              const float coef = chist[ZOH ? t : 0][ZOH ? k : 0];
              const float lB = lam * rec_w[t * R + k];
              dA[k] = __builtin_fmaf(gh, v.x, __builtin_fmaf(lB * v.w, zoh_coef_dA(a, x2, v.x, rA[k]), dA[k]));
              lb = __builtin_fmaf(lB, coef, lb);
              la = __builtin_fmaf(lB, a, la);
              terms[k * TRS + i] = (lam * coef) * v.w;
            } else {
              dA[k] = __builtin_fmaf(gh, v.x, dA[k]);
              lb = __builtin_fmaf(lam, rec_w[t * R + k], lb);
              terms[k * TRS + i] = lam * v.y;
            }
            terms[8 + k * TRS + i] = v.z * hist[t][k];
            carry[k] = cn;
          }
          if constexpr (ZOH) s_p[g][t][lane] = make_float2(lb, __builtin_fmaf(v.w, la, dd * kLn2));
          else s_p[g][t][lane] = make_float2(lb, dd * kLn2);
        }
      }
      // dB, dC of this group's steps: the sums over the 64 channels
      const float sum = wave_sum16(terms, lane);
      // (an ordinary store: these 4-byte pieces of the partial rows merge into
      // whole lines in L2 before they are written back)
      if ((lane & 3) == 0 && (FULL || grp * TRS + so % TRS < tvalid)) pbc[t0 + grp * TRS] = sum;
    }
    __syncthreads();

    // ---- du and d(delta) of this thread's elements -----------------------------------
    float e_du[E], e_dd[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      e_du[e] = e_dd[e] = 0.0f;
      if (e < valid) {
        const int t = r0 + e;
        float slb = 0.0f, sdd = 0.0f;
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
          const float2 q = s_p[gg][t][cc];
          slb += q.x;
          sdd += q.y;
        }
        float ddx;
        if constexpr (ZOH) {  // du = ds D + sum lambda Bbar B; dDelta = u sum lambda Abar B + ...
          e_du[e] = __builtin_fmaf(e_ds[e], D_cc, slb);
          ddx = sdd * e_sg[e];
        } else {              // du = ds D + Delta sum lambda B; dDelta = u sum lambda B + ...
          e_du[e] = __builtin_fmaf(e_ds[e], D_cc, e_dt[e] * slb);
          ddx = __builtin_fmaf(e_u[e], slb, sdd) * e_sg[e];
        }
        e_dd[e] = ddx;
        accD = __builtin_fmaf(e_ds[e], e_u[e], accD);
        accBias += ddx;
      }
    }
    if (valid > 0) {
      if constexpr (FULL) {
        buf_store_run_nt<T, E>(b_du, voff, (uint32_t)t0 * (uint32_t)sizeof(T), e_du);
        buf_store_run_nt<T, E>(b_dd, voff, (uint32_t)t0 * (uint32_t)sizeof(T), e_dd);
      } else {
        store_run<T, E>(du, eoff, vec_ok, valid, e_du);
        store_run<T, E>(ddelta, eoff, vec_ok, valid, e_dd);
      }
    }
  };

  // tiles from last to first: a ragged top tile (or every tile of unaligned
  // rows) on its own path, then the whole tiles, the first of them peeled so
  // that the loop is entered with the same loads in flight as from its back edge
  const int64_t t_top = ((seg_end - 1) / TL) * TL;
  if (!p.vec) {
    for (int64_t t0 = t_top; t0 >= seg_begin; t0 -= TL) tile(BoolC<false>{}, t0, t0);
  } else {
    int64_t t0 = t_top;
    if (seg_end - t_top < TL) {
      tile(BoolC<false>{}, t0, t0);
      t0 -= TL;
    }
    if (t0 >= seg_begin) {
      if constexpr (PF) prefetch(t0);
      tile(BoolC<true>{}, t0, t0 - TL >= seg_begin ? t0 - TL : t0);
      for (int64_t t = t0 - TL; t >= seg_begin; t -= TL) tile(BoolC<true>{}, t, t - TL >= seg_begin ? t - TL : t);
    }
  }

  // ---- per-workgroup results ------------------------------------------------------
#pragma unroll
  for (int off = 1; off < G; off <<= 1) {
    accD += __shfl_xor(accD, off);
    accBias += __shfl_xor(accBias, off);
  }
  if (chunk == 0 && ccvalid) {
    part_d[((int64_t)b * p.nseg + seg) * p.dim + dcc] = accD;
    part_bias[((int64_t)b * p.nseg + seg) * p.dim + dcc] = accBias;
  }
  if (!dvalid) return;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    part_a[(((int64_t)b * p.nseg + seg) * p.dim + d) * N + g * NS + k] = dA[k];
    if (seg == 0 && dh0 != nullptr) dh0[row * N + g * NS + k] = carry[k];
  }
}

// ---- 4. fixed-order sums of the partials ------------------------------------------
// dB, dC: out[w][(b*N + n)*L + t] = sum over channel groups.
template <typename T>
__global__ __launch_bounds__(256) void reduce_bc_kernel(const float* __restrict__ part, T* __restrict__ dB,
                                                        T* __restrict__ dC, int batch, int ncg, int N,
                                                        int64_t L) {
  const int64_t per = (int64_t)N * L;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 * batch * per) return;
  const int w = (int)(i / (batch * per));
  const int64_t j = i % (batch * per);
  const int b = (int)(j / per);
  const int64_t nt = j % per;
  const float* src = part + (((int64_t)b * ncg) * 2 + w) * per + nt;
  float s = 0.0f;
  for (int c = 0; c < ncg; ++c) s += src[(int64_t)c * 2 * per];
  Elem<T>::store((w == 0 ? dB : dC) + j, s);
}

// out[i] = sum_j src[j * n + i], j < terms, for the per-workgroup partials of
// dA, dD and d(bias) (over batch rows and segments), the three in one launch:
// thread i takes element i of the concatenated outputs (a NULL output has
// n = 0 and no elements).
struct TermSums {
  const float* src[3];
  float* out[3];
  int64_t n[3];
};

__global__ __launch_bounds__(256) void reduce_terms_kernel(const TermSums t, int terms) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    if (i < t.n[k]) {
      float s = 0.0f;
      for (int j = 0; j < terms; ++j) s += t.src[k][(int64_t)j * t.n[k] + i];
      t.out[k][i] = s;
      return;
    }
    i -= t.n[k];
  }
}

template <typename T, int NS, int G>
static hipError_t launch_bwd_typed(const BwdLaunch& a, hipStream_t stream) {
  constexpr int TL = kScanTile;
  BwdSizes s;
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
  const T* z = static_cast<const T*>(a.z);
  const T* gy = static_cast<const T*>(a.dy);
  const T* bc = static_cast<const T*>(a.ws_bc);
  const int64_t base = (int64_t)a.batch * s.ncg;
  if (a.nseg > 1) {
    bwd_agg_kernel<T, NS, G, TL><<<(unsigned)(base * (a.nseg - 1)), 64 * G, 0, stream>>>(
        dl, a.A, bc, z, a.bias, gy, a.ws_lagg, a.ws_lsum, s);
  }
  // zero-order hold: half the states per wave, twice the waves (records still
  // in groups of NS)
  constexpr int ZNS = NS >= 2 ? NS / 2 : 1;
  constexpr int ZG = NS * G / ZNS;
  auto kernel = a.zoh ? bwd_kernel<T, ZNS, ZG, TL, true, NS> : bwd_kernel<T, NS, G, TL, false, NS>;
  const int threads = 64 * (a.zoh ? ZG : G);
  kernel<<<(unsigned)(base * a.nseg), threads, 0, stream>>>(
      u, dl, a.A, bc, a.Dskip, z, a.bias, gy, a.dlast, a.ws_ckpt, a.ws_lagg, a.ws_lsum,
      static_cast<T*>(a.du), static_cast<T*>(a.ddelta), static_cast<T*>(a.dz), a.dh0, a.ws_part_bc,
      a.ws_part_a, a.ws_part_d, a.ws_part_bias, s);
  const int N = NS * G;
  const int64_t nbc = 2 * (int64_t)a.batch * N * a.seqlen;
  reduce_bc_kernel<T><<<(unsigned)((nbc + 255) / 256), 256, 0, stream>>>(
      a.ws_part_bc, static_cast<T*>(a.dB), static_cast<T*>(a.dC), a.batch, s.ncg, N, a.seqlen);
  const int terms = a.batch * a.nseg;
  TermSums ts;
  ts.src[0] = a.ws_part_a;
  ts.out[0] = a.dA;
  ts.n[0] = (int64_t)a.dim * N;
  ts.src[1] = a.ws_part_d;
  ts.out[1] = a.dD;
  ts.n[1] = a.dD != nullptr ? a.dim : 0;
  ts.src[2] = a.ws_part_bias;
  ts.out[2] = a.dbias;
  ts.n[2] = a.dbias != nullptr ? a.dim : 0;
  const int64_t nall = ts.n[0] + ts.n[1] + ts.n[2];
  reduce_terms_kernel<<<(unsigned)((nall + 255) / 256), 256, 0, stream>>>(ts, terms);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_bwd_state(const BwdLaunch& a, hipStream_t stream) {
  switch (a.dstate) {
    case 1: return launch_bwd_typed<T, 1, 1>(a, stream);
    case 2: return launch_bwd_typed<T, 2, 1>(a, stream);
    case 4: return launch_bwd_typed<T, 4, 1>(a, stream);
    case 8: return launch_bwd_typed<T, 4, 2>(a, stream);
    case 16: return launch_bwd_typed<T, 4, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scan_bwd(const BwdLaunch& a, hipStream_t stream) {
  if (a.batch == 0 || a.dim == 0 || a.seqlen == 0) return hipSuccess;
  return a.dtype == Dtype::BF16 ? launch_bwd_state<uint16_t>(a, stream)
                                : launch_bwd_state<float>(a, stream);
}

}  // namespace ssm
