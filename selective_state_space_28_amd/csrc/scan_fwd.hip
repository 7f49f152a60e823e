// scan_fwd.hip -- the fused selective-scan forward pass for gfx950.
//
// What it computes is stated in include/ssm.h: per channel (b, d) and state
// n, Delta = softplus(delta + bias), Abar = exp(Delta*A) (zero-order hold,
// "Mamba" paper review, "SSM"), input term Bbar*B*u with Bbar = Delta (the
// Euler form) or, under a flag, (exp(Delta*A) - 1)/A (zero-order hold; both
// in the "Paper: Mamba" course module, "Math & data structures"),
// h = Abar*h + Bbar*B*u, and the readout y = (C.h + D*u)*silu(z) after each
// update ("Exercises -- State-space models (Mamba, S4)", recurrent view).
//
// Design (channel-parallel, one fused pass over HBM):
//  * pack_bc_kernel first rewrites B and C (tiny next to u, delta, z, y:
//    they are shared by all channels) as records, one per (batch row, state
//    group, step) holding that group's B then C values in the input type.
//    In the scan a wave's record for step t is wave-uniform, so it is read
//    with scalar loads into SGPR operands: no VGPRs, no VALU work (a bf16
//    value is widened by a scalar shift or mask).
//  * A workgroup owns 64 consecutive channels of one batch row and G state
//    groups; wave g holds NS = N/G states of each of its 64 channels in
//    VGPRs (lane = channel).  The state never touches HBM.
//  * The sequence is walked in tiles of TL steps, grouped in load blocks of
//    KT tiles whose u, delta (and z) loads are issued together, one block
//    ahead, so each 128-byte line of a row is fetched once.  Per tile, all
//    threads compute Delta = softplus(delta + bias) and Delta*u (u under
//    zero-order hold) once per element and stage them transposed in LDS
//    (one float2 per (step, channel)).
//  * Each wave runs the TL steps of the recurrence for its states: per
//    (element, state) one v_exp_f32 and four fp32 VALU ops (Euler).
//  * The G partial readouts per (step, channel) are summed through LDS in a
//    fixed order, D*u and the silu gate applied, and y kept in registers
//    until the load block ends, then stored so each row line is written
//    whole.
//  * Optional convolution prologue ("Mamba" paper review, "Mamba" block
//    description: before the SSM the input goes through a convolution and
//    then a nonlinear function; NN LAB "Mamba" page, "Kernel Fusion in
//    On-Chip SRAM": a causal 1-D convolution fused with the scan):
//    u = silu(cb + sum_k w[k] x[t-K+1+k]) per channel, computed in the
//    staging step from the loaded x.  The K-1 <= 3 inputs before a thread's
//    run come from the neighbouring run by a lane shuffle (the G runs of a
//    channel sit in consecutive lanes of one wave), or for a channel's
//    first run from the previous tile's last inputs kept in LDS, so x is
//    read from HBM once, as u would be.  The taps also sit in LDS.
//  * Whole load blocks are addressed through buffer descriptors over the
//    workgroup's 64 rows: a lane's offset is fixed, the block's step offset
//    is a scalar, so no lane holds 64-bit addresses.
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
  int ncu;           // compute units of the device (blocks launched per "rank")
  int prio_blocks;   // load blocks per wave-priority step (0: no rotation)
  int conv_k;        // convolution width (CONV variants)
};

// Convolution prologue operands (CONV variants only).
struct ConvArgs {
  const float* w;          // (dim, K)
  const float* b;          // (dim) nullable
  const float* state_in;   // (batch, dim, K-1) nullable: inputs before t = 0
  float* state_out;        // (batch, dim, K-1) nullable: the last K-1 inputs
};

// Input x of row `row` at step s of a sequence of length L: x itself for
// s >= 0, else the carried state (K-1 entries, oldest first) or zero.
template <typename T>
__device__ __forceinline__ float conv_input(const T* __restrict__ x, const float* __restrict__ st,
                                            int64_t row, int64_t L, int64_t s, int K) {
  if (s >= 0) return Elem<T>::load(x + row * L + s);
  if (st != nullptr && s >= -(int64_t)(K - 1)) return st[row * (K - 1) + (K - 1) + s];
  return 0.0f;
}

// ---- B, C -> records (batch, state group, step, [B x NS, C x NS]) -----------
// Records keep the input type: fp32 inputs give fp32 records, bf16 inputs bf16
// records (the same values in half the bytes, so twice the steps per scalar
// cache line).
template <typename T, int NS, int G>
__global__ __launch_bounds__(256) void pack_bc_kernel(const T* __restrict__ B,
                                                      const T* __restrict__ C,
                                                      T* __restrict__ bc, int64_t L,
                                                      int tblocks) {
  constexpr int N = NS * G;
  const int b = blockIdx.x / tblocks;
  const int64_t t = (int64_t)(blockIdx.x % tblocks) * 256 + threadIdx.x;
  if (t >= L) return;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    T v[2 * NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int64_t src = ((int64_t)b * N + g * NS + k) * L + t;
      v[k] = B[src];
      v[NS + k] = C[src];
    }
    T* dst = bc + (((int64_t)b * G + g) * L + t) * (2 * NS);
#pragma unroll
    for (int k = 0; k < 2 * NS; ++k) dst[k] = v[k];
  }
}

// Value q of a record of 2*NS elements starting at p (wave-uniform, so the
// loads are scalar and a bf16 widening is a scalar shift or mask).
template <typename T>
__device__ __forceinline__ float rec_value(const T* __restrict__ p, int q);

template <>
__device__ __forceinline__ float rec_value<float>(const float* __restrict__ p, int q) { return p[q]; }

template <>
__device__ __forceinline__ float rec_value<uint16_t>(const uint16_t* __restrict__ p, int q) {
  const uint32_t w = reinterpret_cast<const uint32_t*>(p)[q >> 1];
  return (q & 1) ? bf16_hi(w) : bf16_lo(w);
}

// Input term of one (element, state).  Euler: q = Delta*u*B is the term.
// Zero-order hold ("Paper: Mamba" course module, "Math & data structures":
// Bbar = (exp(Delta A) - 1)/A B): q = u*B times the coefficient zoh_coef.
template <bool ZOH>
__device__ __forceinline__ float input_term(float a, float x2, float dt, float q, float rA) {
  if constexpr (ZOH) {
    return q * zoh_coef(a, x2, dt, rA);
  } else {
    return q;
  }
}

// PASS: kPassMain computes y (and last_state); kPassAgg runs every segment
// but the last from a zero state and records its end state and Delta sum;
// kPassCkpt runs like the main pass but, instead of y, records the state
// entering every tile (the checkpoints the backward pass starts from);
// kPassMainCkpt computes y and records the checkpoints too.  GATE: the
// passes that compute y apply the silu(z) gate (z given); a compile-time
// choice, so the ungated instantiation carries no gate work and the gated one
// no select.
template <typename T, int NS, int G, int TL, int PASS, int MODE, bool GATE = false>
__global__ __launch_bounds__(64 * G, G == 4 ? 5 : 1) void scan_kernel(
    const T* __restrict__ u, const T* __restrict__ delta, const float* __restrict__ A,
    const T* __restrict__ bc, const float* __restrict__ Dskip, const T* __restrict__ z,
    const float* __restrict__ bias, const float* __restrict__ h0, T* __restrict__ y,
    float* __restrict__ last_state, float* __restrict__ ws_hend, float* __restrict__ ws_sumdt,
    float* __restrict__ ws_ckpt, const ScanSizes p, const ConvArgs cv) {
  constexpr bool AGG = PASS == kPassAgg;
  constexpr bool READOUT = PASS == kPassMain || PASS == kPassMainCkpt;
  constexpr bool CKPT = PASS == kPassCkpt || PASS == kPassMainCkpt;
  constexpr bool ZOH = (MODE & kModeZoh) != 0;
  constexpr bool CONV = (MODE & kModeConv) != 0;
  constexpr int N = NS * G;
  constexpr int E = TL / G;                     // elements per thread, load/store phases
  constexpr int W = E * (int)sizeof(T) / 4;     // their size in 32-bit words
  constexpr int KT = scan_load_block_tiles((int)sizeof(T), G, TL);
  constexpr int LDW = 65;                       // padded LDS row: spreads the banks
  constexpr int CH = 2;                         // steps per software-pipelined chunk
  constexpr int R = 2 * NS;                     // floats per B, C record
  static_assert(TL % G == 0 && (E * (int)sizeof(T)) % 4 == 0, "tile must split into words");
  static_assert(TL % CH == 0, "tile must split into chunks");
  static_assert(!CONV || E >= kMaxConvWidth - 1, "a run must hold the convolution's history");

  __shared__ float2 s_ddu[TL][LDW];                           // (Delta, Delta*u), ZOH: (Delta, u)
  __shared__ float s_y[READOUT ? G : 1][READOUT ? TL : 1][LDW];  // partial readouts
  // convolution taps (right-aligned in 4, tap 3 on the current input) and bias
  // of each channel of the group: read from LDS at each tile's staging rather
  // than held in registers through the whole sequence
  __shared__ float4 s_cw[CONV ? 64 : 1];
  __shared__ float s_cb[CONV ? 64 : 1];
  // the last 3 inputs of each channel's previous tile (convolution halo)
  __shared__ float s_tail[CONV ? kMaxConvWidth - 1 : 1][CONV ? 64 : 1];

  // ---- block -> (batch row, channel group, segment) --------------------------
  // Consecutive block ids go to different XCDs; regroup so that the blocks an
  // XCD runs share batch rows (and hence the B, C records in its L2).  With a
  // single batch row there is nothing to share and the plain order is kept
  // (it measured faster on the split sequence of one row).
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0 && p.batch > 1) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
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

  // step positions fit in 32 bits (the host rejects longer sequences), so the
  // uniform tile bookkeeping stays in scalar registers and scalar compares
  const int seg_begin = seg * (int)p.seglen;
  const int seg_end = (int)min((int64_t)seg_begin + p.seglen, L);

  // ---- per-lane parameters and initial state ---------------------------------
  float A2[NS], h[NS], rA[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const int n = g * NS + k;
    const float a_dn = dvalid ? A[(int64_t)d * N + n] : -1.0f;
    A2[k] = dvalid ? a_dn * kLog2e : 0.0f;
    rA[k] = 1.0f / a_dn;  // zero-order-hold input term only
    h[k] = 0.0f;
    if (seg == 0 && h0 != nullptr && dvalid) h[k] = h0[row * N + n];
  }
  if (!AGG && seg > 0 && dvalid) {
    // carry-in: compose the aggregates of segments 0 .. seg-1 in order.  The
    // aggregates' loads do not depend on the composition, so they are issued
    // in groups whose latencies overlap (indices past seg-1 are clamped to
    // it: in-bounds loads that are not composed).
    constexpr int GRP = 8;
    const int64_t plane = (int64_t)p.batch * p.dim;
#pragma unroll
    for (int k = 0; k < NS; ++k) h[k] = ws_hend[row * N + g * NS + k];
    for (int j0 = 1; j0 < seg; j0 += GRP) {
      float sdt[GRP], he[GRP][NS];
#pragma unroll
      for (int i = 0; i < GRP; ++i) {
        const int j = min(j0 + i, seg - 1);
        sdt[i] = ws_sumdt[j * plane + row];
#pragma unroll
        for (int k = 0; k < NS; ++k) he[i][k] = ws_hend[(j * plane + row) * N + g * NS + k];
      }
#pragma unroll
      for (int i = 0; i < GRP; ++i) {
        if (j0 + i < seg) {
#pragma unroll
          for (int k = 0; k < NS; ++k) h[k] = __builtin_fmaf(segment_decay(sdt[i] * A2[k]), h[k], he[i][k]);
        }
      }
    }
  }

  // ---- load-phase role: thread -> (channel cc, run of E steps) ---------------
  const int cc = tid / G;
  const int chunk = tid % G;
  const int r0 = chunk * E;                 // first step of this thread's run in a tile
  const int dcc = cg * 64 + cc;
  const bool ccvalid = dcc < p.dim;
  const int64_t rowcc = (int64_t)b * p.dim + (ccvalid ? dcc : 0);
  const float bias_cc = (bias != nullptr && ccvalid) ? bias[dcc] : 0.0f;
  const float D_cc = (Dskip != nullptr && ccvalid) ? Dskip[dcc] : 0.0f;
  constexpr bool has_z = READOUT && GATE;
  const bool vec = p.vec != 0;

  if constexpr (CONV) {
    const int K = p.conv_k;
    if (tid < 64) {
      const int dw = cg * 64 + tid;
      float w4[kMaxConvWidth] = {};
      if (dw < p.dim) {
#pragma unroll
        for (int j = 0; j < kMaxConvWidth; ++j) {
          const int k = j - (kMaxConvWidth - K);
          if (k >= 0) w4[j] = cv.w[(int64_t)dw * K + k];
        }
      }
      s_cw[tid] = make_float4(w4[0], w4[1], w4[2], w4[3]);
      s_cb[tid] = (dw < p.dim && cv.b != nullptr) ? cv.b[dw] : 0.0f;
    }
    if (tid < 64) {
      // before the segment's first tile, the "previous tile" ends at the
      // segment start
      const int dw = cg * 64 + tid;
      const int64_t roww = (int64_t)b * p.dim + (dw < p.dim ? dw : 0);
#pragma unroll
      for (int i = 0; i < kMaxConvWidth - 1; ++i)
        s_tail[i][tid] = dw < p.dim ? conv_input<T>(u, cv.state_in, roww, L, seg_begin - (kMaxConvWidth - 1) + i, K)
                                    : 0.0f;
    }
    __syncthreads();
  }

  const T* bcw = bc + ((int64_t)b * G + g) * L * R;  // wave-uniform records

  // Whole load blocks go through buffer descriptors over the workgroup's rows
  // of u, delta, z and y: a lane's offset (channel cc, step r0) is fixed and
  // the block's step offset is a scalar, so no lane holds 64-bit addresses.
  // Rows past dim lie beyond the extent: they read 0 and their stores drop.
  // (vec is set only when the rows of 64 channels span < 2^31 bytes.)
  const int64_t grow = (int64_t)b * p.dim + (int64_t)cg * 64;
  const int64_t gbytes = (int64_t)min(64, p.dim - cg * 64) * L * (int64_t)sizeof(T);
  const Buf bu = make_buf(u + grow * L, vec ? gbytes : 0);
  const Buf bd = make_buf(delta + grow * L, vec ? gbytes : 0);
  const Buf bz = make_buf(has_z ? z + grow * L : u, (vec && has_z) ? gbytes : 0);
  const Buf by = make_buf(READOUT ? y + grow * L : u, (vec && READOUT) ? gbytes : 0);
  const uint32_t voff = vec ? (uint32_t)(((int64_t)cc * L + r0) * (int64_t)sizeof(T)) : 0u;

  // raw words of this thread's runs in the KT tiles of the current load block,
  // and the packed y of those runs, stored together at the end of the block
  // so each 128-byte row line is written whole
  uint32_t pu[KT][W], pd[KT][W], pz[KT][W], py[KT][W];
  auto block_full = [&](int tb) { return vec && tb + KT * TL <= seg_end; };
  auto fetch_block = [&](int tb) {
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const uint32_t soff = (uint32_t)(tb + j * TL) * (uint32_t)sizeof(T);
      buf_load_words<W>(bu, voff, soff, pu[j]);
      buf_load_words<W>(bd, voff, soff, pd[j]);
      if (has_z) buf_load_words<W>(bz, voff, soff, pz[j]);
    }
  };
  if (block_full(seg_begin)) fetch_block(seg_begin);

  // Delta sum of this thread's runs (aggregate pass), gathered in the staging
  // step, which every wave shares evenly, and reduced over a channel's G
  // threads at the end
  double sumdt = 0.0;

  // The wave arbiter prefers older waves, so of the workgroups resident on a
  // CU the oldest ones would race ahead and the youngest run alone at the
  // end, unable to fill the SIMDs.  Blocks are dispatched round-robin over
  // the CUs, so blockIdx / ncu is a block's age rank on its CU; rotating a
  // raised wave priority over the ranks keeps them progressing together; the
  // priorities move on every prio_blocks load blocks (every block by default:
  // the tighter the rotation, the closer together the ranks finish).
  const int prio_rank = (int)(blockIdx.x / (unsigned)p.ncu) % 5;
  const int epoch_len = p.prio_blocks;

  // One tile of TL steps.  FAST: a whole tile of a whole load block, its runs
  // already in registers (pu, pd, pz) and its y packed into py; otherwise a
  // ragged or unaligned tile with element loads and guards.
  auto tile = [&](auto fast_c, int j, int tb, int t0, int tvalid) {
    constexpr bool FAST = decltype(fast_c)::value;
    // ---- this tile's u, delta (z) -> Delta, Delta*u in LDS --------------------
    float uu[E], dd[E], zz[E];
    if constexpr (FAST) {
      words_to_floats<T, E>(pu[j], uu);
      words_to_floats<T, E>(pd[j], dd);
      if (has_z) words_to_floats<T, E>(pz[j], zz);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool ok = ccvalid && r0 + e < tvalid;
        const int64_t off = rowcc * L + t0 + r0 + e;
        uu[e] = ok ? Elem<T>::load(u + off) : 0.0f;
        dd[e] = ok ? Elem<T>::load(delta + off) : 0.0f;
        zz[e] = (ok && has_z) ? Elem<T>::load(z + off) : 0.0f;
      }
    }
    float xlast[kMaxConvWidth - 1] = {};  // this run's last 3 inputs (convolution)
    if constexpr (CONV) {
#pragma unroll
      for (int i = 0; i < kMaxConvWidth - 1; ++i) xlast[i] = uu[E - (kMaxConvWidth - 1) + i];
      // the 3 inputs before this run: from the run of the lane before (same
      // tile, a lane shuffle), or for a channel's first run from the last 3
      // inputs of the previous tile, which that tile's last run left in LDS
      // (written before two barriers, read after them)
      const int lw = tid & 63;
      float xw[E + kMaxConvWidth - 1];
#pragma unroll
      for (int i = 0; i < kMaxConvWidth - 1; ++i) {
        const float left = __shfl(uu[E - (kMaxConvWidth - 1) + i], chunk > 0 ? lw - 1 : lw);
        xw[i] = chunk > 0 ? left : s_tail[i][cc];
      }
#pragma unroll
      for (int e = 0; e < E; ++e) xw[kMaxConvWidth - 1 + e] = uu[e];
      const float4 w4 = s_cw[cc];
      const float cw[kMaxConvWidth] = {w4.x, w4.y, w4.z, w4.w};
      const float cbias = s_cb[cc];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float sacc = cbias;
#pragma unroll
        for (int q = 0; q < kMaxConvWidth; ++q) sacc = __builtin_fmaf(cw[q], xw[e + q], sacc);
        uu[e] = silu_f32(sacc);
      }
    }
    // Entries of channels past dim, or of steps past the tile end, hold
    // harmless values (u = 0 there, so Delta*u = 0): those steps are never
    // run and those lanes never store.
    float dsum = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float x = dd[e] + bias_cc;
      const float dt = p.softplus ? softplus_f32(x) : x;
      s_ddu[r0 + e][cc] = make_float2(dt, ZOH ? uu[e] : dt * uu[e]);
      if constexpr (AGG) {
        if (FAST || r0 + e < tvalid) dsum += dt;
      }
    }
    if constexpr (AGG) sumdt += (double)dsum;
    __syncthreads();
    if constexpr (CONV) {
      // this tile's last 3 inputs for the next tile (the reads above of the
      // previous tile's are ordered before this by the barrier)
      if (chunk == G - 1) {
#pragma unroll
        for (int i = 0; i < kMaxConvWidth - 1; ++i) s_tail[i][cc] = xlast[i];
      }
    }

    // ---- after the block's last tile is staged, issue the next block --------
    if (FAST && j == KT - 1) {
      const int tn = tb + KT * TL;
      if (block_full(tn)) fetch_block(tn);
    }

    // ---- checkpoint: the state entering this tile, (batch, tile, N, dim) ------
    // (non-temporal: read once, by the backward pass, long after this pass)
    if constexpr (CKPT) {
      if (dvalid) {
        const int64_t ntiles = (L + TL - 1) / TL;
        float* cp = ws_ckpt + (((int64_t)b * ntiles + t0 / TL) * N + g * NS) * p.dim + d;
#pragma unroll
        for (int k = 0; k < NS; ++k) __builtin_nontemporal_store(h[k], cp + (int64_t)k * p.dim);
      }
    }

    // ---- the recurrence: TL steps x NS states per lane -----------------------
    const T* bct = bcw + (int64_t)t0 * R;
    if (FAST || tvalid == TL) {
      // chunks of CH steps; the next chunk's LDS and scalar loads are issued
      // before the current chunk's arithmetic so their latency is covered
      float2 vc[CH], vn[CH];
      float rc[CH][R], rn[CH][R];
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        vc[i] = s_ddu[i][lane];
#pragma unroll
        for (int q = 0; q < R; ++q) rc[i][q] = rec_value<T>(bct + i * R, q);
      }
#pragma unroll
      for (int c = 0; c < TL / CH; ++c) {
        if (c + 1 < TL / CH) {
#pragma unroll
          for (int i = 0; i < CH; ++i) {
            vn[i] = s_ddu[(c + 1) * CH + i][lane];
#pragma unroll
            for (int q = 0; q < R; ++q) rn[i][q] = rec_value<T>(bct + ((c + 1) * CH + i) * R, q);
          }
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          float acc = 0.0f;
#pragma unroll
          for (int k = 0; k < NS; ++k) {
            const float x2 = vc[i].x * A2[k];
            const float a = exp2_hw(x2);
            h[k] = __builtin_fmaf(a, h[k], input_term<ZOH>(a, x2, vc[i].x, vc[i].y * rc[i][k], rA[k]));
            acc = __builtin_fmaf(rc[i][NS + k], h[k], acc);
          }
          if constexpr (READOUT) s_y[g][c * CH + i][lane] = acc;
        }
        if (c + 1 < TL / CH) {
#pragma unroll
          for (int i = 0; i < CH; ++i) {
            vc[i] = vn[i];
#pragma unroll
            for (int q = 0; q < R; ++q) rc[i][q] = rn[i][q];
          }
        }
      }
    } else {
      for (int t = 0; t < tvalid; ++t) {
        const float2 v = s_ddu[t][lane];
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < NS; ++k) {
          const float x2 = v.x * A2[k];
          const float a = exp2_hw(x2);
          h[k] = __builtin_fmaf(a, h[k], input_term<ZOH>(a, x2, v.x, v.y * rec_value<T>(bct + t * R, k), rA[k]));
          acc = __builtin_fmaf(rec_value<T>(bct + t * R, NS + k), h[k], acc);
        }
        if constexpr (READOUT) s_y[g][t][lane] = acc;
      }
    }
    __syncthreads();

    // ---- readout: sum the G partials, D-skip, gate, store y --------------------
    if constexpr (READOUT) {
      float yv[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float sum = s_y[0][r0 + e][cc];
#pragma unroll
        for (int gg = 1; gg < G; ++gg) sum += s_y[gg][r0 + e][cc];
        sum = __builtin_fmaf(D_cc, uu[e], sum);
        if (has_z) sum *= silu_f32(zz[e]);
        yv[e] = sum;
      }
      if constexpr (FAST) {
        // rows past dim are beyond the buffer's extent: their stores drop
        pack_floats<T, E>(yv, py[j]);
        if (j == KT - 1) {
#pragma unroll
          for (int jj = 0; jj < KT; ++jj)
            buf_store_words<W>(by, voff, (uint32_t)(tb + jj * TL) * (uint32_t)sizeof(T), py[jj]);
        }
      } else if (ccvalid) {
        const int64_t off = rowcc * L + t0 + r0;
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (r0 + e < tvalid) Elem<T>::store(y + off + e, yv[e]);
      }
    }
    // The next tile's LDS writes (s_ddu) are not read by this readout, and its
    // s_y writes come after the next barrier, so no third barrier is needed.
  };

  int blk = 0;
  for (int tb = seg_begin; tb < seg_end; tb += KT * TL, ++blk) {
    if (epoch_len > 0 && blk % epoch_len == 0) {
      const int lvl = (prio_rank + blk / epoch_len) % 5;
      if (lvl <= 1) __builtin_amdgcn_s_setprio(0);
      else if (lvl == 2) __builtin_amdgcn_s_setprio(1);
      else if (lvl == 3) __builtin_amdgcn_s_setprio(2);
      else __builtin_amdgcn_s_setprio(3);
    }
    const bool fast = block_full(tb);
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      const int t0 = tb + j * TL;
      if (t0 >= seg_end) break;
      if (fast) tile(BoolC<true>{}, j, tb, t0, TL);
      else tile(BoolC<false>{}, j, tb, t0, min(TL, seg_end - t0));
    }
  }

  // ---- segment results ---------------------------------------------------------
  if constexpr (AGG) {
    // a channel's G staging threads are consecutive lanes of one wave: sum
    // their Delta sums in a fixed order (every lane takes part)
#pragma unroll
    for (int m = 1; m < G; m <<= 1) sumdt += __shfl_xor(sumdt, m);
    if (chunk == 0 && ccvalid) ws_sumdt[(int64_t)seg * p.batch * p.dim + rowcc] = (float)sumdt;
  }
  if (!dvalid) return;
  if constexpr (AGG) {
    const int64_t plane = (int64_t)p.batch * p.dim;
#pragma unroll
    for (int k = 0; k < NS; ++k) ws_hend[(seg * plane + row) * N + g * NS + k] = h[k];
  } else if constexpr (READOUT) {
    if (last_state != nullptr && seg == p.nseg - 1) {
#pragma unroll
      for (int k = 0; k < NS; ++k) last_state[row * N + g * NS + k] = h[k];
    }
    if constexpr (CONV) {
      if (cv.state_out != nullptr && seg == p.nseg - 1 && g == 0) {
        const int K = p.conv_k;
        for (int j = 0; j < K - 1; ++j)
          cv.state_out[row * (K - 1) + j] = conv_input<T>(u, cv.state_in, row, L, L - (K - 1) + j, K);
      }
    }
  }
}

template <typename T, int NS, int G, int MODE>
static hipError_t launch_typed(const ScanLaunch& a, hipStream_t stream) {
  constexpr int TL = kScanTile;
  const T* B = static_cast<const T*>(a.B);
  const T* C = static_cast<const T*>(a.C);
  const int tblocks = (int)((a.seqlen + 255) / 256);
  T* bc = static_cast<T*>(a.ws_bc);
  pack_bc_kernel<T, NS, G><<<(unsigned)((int64_t)a.batch * tblocks), 256, 0, stream>>>(
      B, C, bc, a.seqlen, tblocks);

  ScanSizes s;
  s.batch = a.batch;
  s.dim = a.dim;
  s.seqlen = a.seqlen;
  s.seglen = a.seglen;
  s.nseg = a.nseg;
  s.ncg = (a.dim + 63) / 64;
  s.softplus = a.softplus;
  s.vec = a.vec;
  s.ncu = a.ncu > 0 ? a.ncu : 1;
  s.prio_blocks = a.prio_blocks;
  s.conv_k = a.conv_k;
  const ConvArgs cv{a.conv_w, a.conv_b, a.conv_state_in, a.conv_state_out};
  const T* u = static_cast<const T*>(a.u);
  const T* dl = static_cast<const T*>(a.delta);
  const T* z = static_cast<const T*>(a.z);
  T* y = static_cast<T*>(a.y);
  const int64_t base = (int64_t)a.batch * s.ncg;
  if (a.nseg > 1) {
    s.nseg_launch = a.nseg - 1;
    const unsigned grid = (unsigned)(base * s.nseg_launch);
    // the aggregate pass has no readout: with 16 states it takes 32-step
    // tiles, half the barriers per step (same load blocks, so the same
    // segment granule)
    constexpr int TLA = G == 4 ? 2 * TL : TL;
    static_assert(scan_load_block_tiles((int)sizeof(T), G, TLA) * TLA ==
                      scan_load_block_tiles((int)sizeof(T), G, TL) * TL,
                  "the aggregate and main passes share the load-block granule");
    scan_kernel<T, NS, G, TLA, kPassAgg, MODE><<<grid, 64 * G, 0, stream>>>(
        u, dl, a.A, bc, a.Dskip, z, a.bias, a.h0, y, a.last_state, a.ws_hend, a.ws_sumdt, nullptr,
        s, cv);
  }
  s.nseg_launch = a.nseg;
  const unsigned grid = (unsigned)(base * s.nseg_launch);
  if constexpr ((MODE & kModeConv) == 0) {  // the backward pass covers both input terms, no prologue
    if (a.ws_ckpt != nullptr && a.ckpt_with_y) {
      auto kernel = z != nullptr ? scan_kernel<T, NS, G, TL, kPassMainCkpt, MODE, true>
                                 : scan_kernel<T, NS, G, TL, kPassMainCkpt, MODE, false>;
      kernel<<<grid, 64 * G, 0, stream>>>(u, dl, a.A, bc, a.Dskip, z, a.bias, a.h0, y, a.last_state,
                                          a.ws_hend, a.ws_sumdt, a.ws_ckpt, s, cv);
      return hipGetLastError();
    }
    if (a.ws_ckpt != nullptr) {
      scan_kernel<T, NS, G, TL, kPassCkpt, MODE><<<grid, 64 * G, 0, stream>>>(
          u, dl, a.A, bc, a.Dskip, z, a.bias, a.h0, y, a.last_state, a.ws_hend, a.ws_sumdt,
          a.ws_ckpt, s, cv);
      return hipGetLastError();
    }
  }
  auto kernel = z != nullptr ? scan_kernel<T, NS, G, TL, kPassMain, MODE, true>
                             : scan_kernel<T, NS, G, TL, kPassMain, MODE, false>;
  kernel<<<grid, 64 * G, 0, stream>>>(u, dl, a.A, bc, a.Dskip, z, a.bias, a.h0, y, a.last_state,
                                      a.ws_hend, a.ws_sumdt, nullptr, s, cv);
  return hipGetLastError();
}

template <typename T, int NS, int G>
static void pack_only(const ScanLaunch& a, hipStream_t stream) {
  const int tblocks = (int)((a.seqlen + 255) / 256);
  pack_bc_kernel<T, NS, G><<<(unsigned)((int64_t)a.batch * tblocks), 256, 0, stream>>>(
      static_cast<const T*>(a.B), static_cast<const T*>(a.C), static_cast<T*>(a.ws_bc), a.seqlen,
      tblocks);
}

template <typename T>
static hipError_t pack_by_state(const ScanLaunch& a, hipStream_t stream) {
  switch (a.dstate) {
    case 1: pack_only<T, 1, 1>(a, stream); break;
    case 2: pack_only<T, 2, 1>(a, stream); break;
    case 4: pack_only<T, 4, 1>(a, stream); break;
    case 8: pack_only<T, 4, 2>(a, stream); break;
    case 16: pack_only<T, 4, 4>(a, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int MODE>
static hipError_t launch_by_state(const ScanLaunch& a, hipStream_t stream) {
  switch (a.dstate) {
    case 1: return launch_typed<T, 1, 1, MODE>(a, stream);
    case 2: return launch_typed<T, 2, 1, MODE>(a, stream);
    case 4: return launch_typed<T, 4, 1, MODE>(a, stream);
    case 8: return launch_typed<T, 4, 2, MODE>(a, stream);
    case 16: return launch_typed<T, 4, 4, MODE>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t launch_by_mode(const ScanLaunch& a, hipStream_t stream) {
  const int mode = (a.zoh ? kModeZoh : 0) | (a.conv_w != nullptr ? kModeConv : 0);
  switch (mode) {
    case 0: return launch_by_state<T, 0>(a, stream);
    case kModeZoh: return launch_by_state<T, kModeZoh>(a, stream);
    case kModeConv: return launch_by_state<T, kModeConv>(a, stream);
    default: return launch_by_state<T, kModeZoh | kModeConv>(a, stream);
  }
}

hipError_t launch_scan_fwd(const ScanLaunch& a, hipStream_t stream) {
  if (a.batch == 0 || a.dim == 0 || a.seqlen == 0) return hipSuccess;
  if (a.conv_w != nullptr && (a.conv_k < 1 || a.conv_k > kMaxConvWidth)) return hipErrorInvalidValue;
  if (a.ws_ckpt != nullptr && a.conv_w != nullptr) return hipErrorInvalidValue;
  return a.dtype == Dtype::BF16 ? launch_by_mode<uint16_t>(a, stream) : launch_by_mode<float>(a, stream);
}

hipError_t launch_pack_records(const ScanLaunch& a, hipStream_t stream) {
  if (a.batch == 0 || a.seqlen == 0) return hipSuccess;
  return a.dtype == Dtype::BF16 ? pack_by_state<uint16_t>(a, stream) : pack_by_state<float>(a, stream);
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
