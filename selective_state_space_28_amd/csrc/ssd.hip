// ssd.hip -- the SSD (Mamba-2) form of the selective scan for gfx950: a
// scalar A per head, evaluated by chunks on the matrix cores.
//
// With A = alpha I ("Mamba" paper review, "Mamba 2"; NN LAB "Mamba" page,
// "Bridging Tensor Cores and Recurrence") the scan of a head is y = M x with
// M[t, s] = C_t . B_s * prod_{s<k<=t} Abar_k * Bbar_s: within a chunk a
// masked matrix product (the quadratic form), across chunks a linear
// recurrence of an N x P state.  Per chunk of Q = 64 steps and head h
// (P = 64 channels, N states), with cum_t the inclusive sum of Delta A over
// the chunk:
//
//   G     = C^T B                                (Q x Q,  K = N)
//   M     = G o exp(cum_t - cum_s) Bbar_s, s <= t
//   Y     = M X^T + diag(exp(cum_t)) C^T H        (Q x P,  K = Q and K = N)
//   H    <- exp(cum_Q) H + (B o exp(cum_Q - cum_s) Bbar_s) X^T   (N x P, K = Q)
//
// then y = Y + D x, times silu(z).  G does not depend on the head: a prep
// kernel forms its causal tiles once per (batch row, chunk), with C^T, into
// the workspace.  Then one workgroup (4 waves) owns a (batch row, head) and
// walks its chunks in order; H never leaves the matrix-core accumulators
// (registers), so HBM sees x, delta, z and y once, and B, C^T and G once per
// XCD that runs the row's heads.  Bbar_s is Delta_s (Euler) or
// (exp(Delta_s A) - 1)/A (zero-order hold), as in the diagonal scan.
#include "ssm_kernels.hpp"
#include "ssm_math.hpp"

namespace ssm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Matrix-core operand traits.  One 16x16 output tile, K per instruction:
// lane l supplies A[l % 16][k0 + KL * (l / 16) + j] and B[k0 + KL * (l / 16) + j][l % 16]
// (j < KL) and receives D[4 * (l / 16) + i][l % 16] (i < 4).
template <typename T>
struct Mma;

template <>
struct Mma<uint16_t> {  // bf16 storage: bf16 operands, v_mfma_f32_16x16x32_bf16
  using Op = __bf16;
  static constexpr int KL = 8;
  static constexpr int K = 32;
  __device__ static f32x4_t mma(const Op* a, const Op* b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8_t*>(a),
                                                   *reinterpret_cast<const bf16x8_t*>(b), c, 0, 0,
                                                   0);
  }
  __device__ static Op cvt(float v) { return (__bf16)v; }
  // Products with the state H (N x 16 channels, held as 16x16 accumulator
  // tiles: lane l has states 16k + 4*(l/16) + i, channel l % 16) contract over
  // the state index.  One instruction takes 32 states as K: lane l's 8 B
  // values are its accumulator rows of two tiles (states 32m + 4*(l/16) + i
  // and 32m + 16 + 4*(l/16) + i), so the A operand (C^T, B^T) is staged in LDS
  // with the states of each 32-block in that order: state_pos(n).
  static constexpr int kPackStates = 32;
  __device__ static int state_pos(int n) {
    const int q = n & 31;
    return (n & ~31) + 8 * ((q & 15) >> 2) + 4 * (q >> 4) + (q & 3);
  }
  using StatePack = bf16x8_t;
  __device__ static StatePack pack_state(f32x4_t lo, f32x4_t hi) {
    StatePack v;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = (__bf16)lo[j];
      v[4 + j] = (__bf16)hi[j];
    }
    return v;
  }
  // acc += A (16 rows of a [.][lda] array at a, 32 staged states) times the pack
  __device__ static f32x4_t mma_state(const Op* a, int lda, StatePack b, f32x4_t acc, int lane) {
    const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(a + (lane & 15) * lda + 8 * (lane >> 4));
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b, acc, 0, 0, 0);
  }
};

template <>
struct Mma<float> {  // fp32 storage: fp32 operands, v_mfma_f32_16x16x4_f32
  using Op = float;
  static constexpr int KL = 1;
  static constexpr int K = 4;
  __device__ static f32x4_t mma(const Op* a, const Op* b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(*a, *b, c, 0, 0, 0);
  }
  __device__ static Op cvt(float v) { return v; }
  // products with the state: one 16-state tile per pack, states in natural
  // order, as four K = 4 products (the r-th takes state 4 * (l/16) + r from
  // each lane's own accumulator element r)
  static constexpr int kPackStates = 16;
  __device__ static int state_pos(int n) { return n; }
  using StatePack = f32x4_t;
  __device__ static StatePack pack_state(f32x4_t lo, f32x4_t) { return lo; }
  __device__ static f32x4_t mma_state(const Op* a, int lda, StatePack b, f32x4_t acc, int lane) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[(lane & 15) * lda + 4 * (lane >> 4) + r], b[r], acc, 0,
                                                  0, 0);
    return acc;
  }
};

struct SsdSizes {
  int batch, nheads;
  int64_t seqlen;
  int softplus, zoh, vec;
};

// One 16x16 tile of A (rows r0.., row-major, leading dimension lda) times B
// stored transposed (cols c0.., each column's K values contiguous, ldb),
// over k in [0, kdim): acc += A B.
template <typename T>
__device__ __forceinline__ f32x4_t tile_mma(const typename Mma<T>::Op* A, int lda, int r0,
                                            const typename Mma<T>::Op* Bt, int ldb, int c0, int kdim,
                                            int lane, f32x4_t acc) {
  using M = Mma<T>;
  const int rr = lane & 15;
  const int kk = M::KL * (lane >> 4);
#pragma unroll
  for (int k0 = 0; k0 < kdim; k0 += M::K)
    acc = M::mma(A + (r0 + rr) * lda + k0 + kk, Bt + (c0 + rr) * ldb + k0 + kk, acc);
  return acc;
}

// Words of a run of 8 consecutive elements of T.
template <typename T>
constexpr int kRunWords = 8 * (int)sizeof(T) / 4;

// 8 elements at p into raw words: one or two 16-byte loads when `vec`, else
// element loads with zeros past `valid`.
template <typename T>
__device__ __forceinline__ void load_run8(const T* __restrict__ p, bool vec, int valid,
                                          uint32_t (&w)[kRunWords<T>]) {
  if (vec) {
    load_words<kRunWords<T>>(p, w);
  } else if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = 2 * q < valid ? (uint32_t)p[2 * q] : 0u;
      const uint32_t hi = 2 * q + 1 < valid ? (uint32_t)p[2 * q + 1] : 0u;
      w[q] = lo | (hi << 16);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = q < valid ? __float_as_uint(p[q]) : 0u;
  }
}

// Buffer accesses (Buf, make_buf in ssm_math.hpp): a descriptor per block
// region, a 32-bit per-lane offset that stays fixed from chunk to chunk and a
// scalar offset that moves with the chunk.  Extents are below 2^31 bytes
// (checked on the host).

// A run of 8 elements of T (16 or 32 bytes) at voff + soff.
template <typename T>
__device__ __forceinline__ void buf_load_run8(const Buf& b, uint32_t voff, uint32_t soff,
                                              uint32_t (&w)[kRunWords<T>]) {
#pragma unroll
  for (int i = 0; i < kRunWords<T> / 4; ++i) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(b.r, voff + 16 * i, soff, 0);
    w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
  }
}

// A run of 4 elements of T (8 or 16 bytes) at voff + soff.
template <typename T>
__device__ __forceinline__ void buf_load_run4(const Buf& b, uint32_t voff, uint32_t soff,
                                              uint32_t (&w)[kRunWords<T> / 2]) {
  if constexpr (sizeof(T) == 2) {
    const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(b.r, voff, soff, 0);
    w[0] = v.x; w[1] = v.y;
  } else {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(b.r, voff, soff, 0);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
}

__device__ __forceinline__ float4 buf_load_f4(const Buf& b, uint32_t voff, uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(b.r, voff, soff, 0);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

__device__ __forceinline__ void buf_load_elem(const Buf& b, uint32_t voff, uint32_t soff, uint16_t& v) {
  v = __builtin_amdgcn_raw_buffer_load_b16(b.r, voff, soff, 0);
}
__device__ __forceinline__ void buf_load_elem(const Buf& b, uint32_t voff, uint32_t soff, float& v) {
  v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(b.r, voff, soff, 0));
}

// A raw element as float.
__device__ __forceinline__ float raw_value(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ float raw_value(float v) { return v; }

// Run j of the transpose of an 8 x 8 tile (rows i = 0..7, each a run of 8):
// (tile[0][j], ..., tile[7][j]) as raw words.
template <typename T>
__device__ __forceinline__ void tile_column(const uint32_t (&tile)[8][kRunWords<T>], int j,
                                            uint32_t (&out)[kRunWords<T>]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t a = tile[2 * q][j >> 1], b = tile[2 * q + 1][j >> 1];
      out[q] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = tile[i][j];
  }
}

// Element j (0..3) of a 4-element run, as float.
template <typename T>
__device__ __forceinline__ float run_elem4(const uint32_t (&w)[kRunWords<T> / 2], int j) {
  if constexpr (sizeof(T) == 2) return (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
  else return __uint_as_float(w[j]);
}

// Element j (0..7) of a run, as float.
template <typename T>
__device__ __forceinline__ float run_elem(const uint32_t (&w)[kRunWords<T>], int j) {
  if constexpr (sizeof(T) == 2) return (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
  else return __uint_as_float(w[j]);
}

template <typename T>
__device__ __forceinline__ void lds_store_run(void* dst, const uint32_t (&w)[kRunWords<T>]) {
  store_words<kRunWords<T>>(dst, w);
}

// A run of 8 consecutive states (n8..n8+7, n8 a multiple of 8) into a row of
// state-staged operands: bf16 splits it into two 4-state pieces.
template <typename T>
__device__ __forceinline__ void lds_store_states(typename Mma<T>::Op* row, int n8,
                                                 const uint32_t (&w)[kRunWords<T>]) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t lo[2] = {w[0], w[1]}, hi[2] = {w[2], w[3]};
    store_words<2>(row + Mma<T>::state_pos(n8), lo);
    store_words<2>(row + Mma<T>::state_pos(n8 + 4), hi);
  } else {
    store_words<kRunWords<T>>(row + n8, w);
  }
}


// The 10 causal 16x16 tiles (t-block i, s-block j <= i) of a 64-step chunk
// matrix, numbered row by row: tile q has i = the largest with i(i+1)/2 <= q.
__device__ __forceinline__ int causal_tile_row(int q) { return q < 1 ? 0 : q < 3 ? 1 : q < 6 ? 2 : 3; }

// The k-th (k < 3) causal tile that wave w (w < 4) forms in the scan, or -1:
// one diagonal tile per wave (0, 5, 2, 9; the costly ones, with a decay per
// entry) as k = 0, then the ones below the diagonal as k = 1, 2 (the mask
// step relies on this order).
__device__ __forceinline__ int wave_mask_tile(int w, int k) {
  const int t0 = w == 0 ? 0 : w == 1 ? 5 : w == 2 ? 2 : 9;
  const int t1 = w == 0 ? 4 : w == 1 ? 1 : w == 2 ? 6 : 3;
  const int t2 = w == 0 ? 8 : w == 1 ? 7 : -1;
  return k == 0 ? t0 : k == 1 ? t1 : t2;
}

// Per (batch row, chunk of 64 steps): C^T with the state index contiguous,
// (batch, L, N), for the products with the state, and the chunk's causal
// tiles of G = C^T B (G[t][s] = C_t . B_s), which do not depend on the head:
// formed once here for every head of the row.  Tile q is stored as 64 lanes x
// 4 floats, lane l holding G[16i + l % 16][16j + 4 (l / 16) + r], r < 4 -- the
// order in which the scan's lanes use it.
template <typename T, int N>
__global__ __launch_bounds__(256) void ssd_prep_kernel(const T* __restrict__ B, const T* __restrict__ C,
                                                       T* __restrict__ Ct, float4* __restrict__ G,
                                                       int64_t L, int nchunks, int vec) {
  using Op = typename Mma<T>::Op;
  constexpr int KN = (N + Mma<T>::K - 1) / Mma<T>::K * Mma<T>::K;
  constexpr int LN = KN + 16 / (int)sizeof(Op);
  __shared__ __align__(16) Op sBt[64][LN];   // [s][n]
  __shared__ __align__(16) Op sCt[64][LN];   // [t][n]
  // the same regrouping over XCDs as the scan, so a batch row's C^T and tiles
  // are written from the XCD whose L2 will read them
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int b = bid / nchunks;
  const int c = bid % nchunks;
  const int64_t t0 = (int64_t)c * 64;
  const T* Bb = B + (int64_t)b * N * L;
  const T* Cb = C + (int64_t)b * N * L;
  // Staging: item q takes an 8 x 8 tile (states n0..n0+7, steps t8..t8+7) of
  // B (q < N) or C: 8 runs of 8 steps read from the (N, L) rows, turned in
  // registers into 8 runs of 8 states, one per step, each written whole.
  // Consecutive items take consecutive state tiles of one step tile, so the
  // lanes of an LDS write phase fill one contiguous row segment.  Steps past
  // the sequence are zeros.
  constexpr int RW = kRunWords<T>;
  const bool whole = vec && t0 + 64 <= L;  // every run 16-byte aligned and inside the sequence
  for (int q = threadIdx.x; q < 2 * N; q += 256) {
    const int which = q / N, r = q % N;
    const int n0 = 8 * (r % (N / 8)), t8 = 8 * (r / (N / 8));
    const T* src = (which == 0 ? Bb : Cb) + (int64_t)n0 * L + t0 + t8;
    const int valid = (int)(L - t0) - t8;  // steps of these runs inside the sequence (any sign)
    uint32_t tile[8][RW];
#pragma unroll
    for (int i = 0; i < 8; ++i) load_run8<T>(src + (int64_t)i * L, whole, valid, tile[i]);
    Op(*dst)[LN] = which == 0 ? sBt : sCt;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t col[RW];
      tile_column<T>(tile, j, col);
      store_words<RW>(&dst[t8 + j][n0], col);
    }
  }
  if constexpr (KN > N) {  // the padded states stay zero
    for (int i = threadIdx.x; i < 64 * (KN - N); i += 256) {
      sBt[i / (KN - N)][N + i % (KN - N)] = Mma<T>::cvt(0.0f);
      sCt[i / (KN - N)][N + i % (KN - N)] = Mma<T>::cvt(0.0f);
    }
  }
  __syncthreads();
  T* Ctb = Ct + ((int64_t)b * L + t0) * N;
  for (int i = threadIdx.x; i < 64 * (N / 8); i += 256) {
    const int tt = i / (N / 8), n8 = 8 * (i % (N / 8));
    if (t0 + tt < L) {
      uint32_t w[RW];
      load_words<RW>(&sCt[tt][n8], w);
      store_words<RW>(Ctb + (int64_t)tt * N + n8, w);
    }
  }
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int q = w; q < 10; q += 4) {
    const int i = causal_tile_row(q), j = q - i * (i + 1) / 2;
    f32x4_t g = {0.0f, 0.0f, 0.0f, 0.0f};
    g = tile_mma<T>(&sBt[0][0], LN, 16 * j, &sCt[0][0], LN, 16 * i, KN, lane, g);
    G[(((int64_t)b * nchunks + c) * 10 + q) * 64 + lane] = make_float4(g[0], g[1], g[2], g[3]);
  }
}

// Eight bf16 operand values of a lane from LDS (one 16-byte read).
__device__ __forceinline__ bf16x8_t lds_frag8(const __bf16* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within each row of
// 16 lanes, then the row totals carried forward by row broadcasts.
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += dpp_moved<0x111, 0xf>(v);  // row_shr:1
  v += dpp_moved<0x112, 0xf>(v);  // row_shr:2
  v += dpp_moved<0x114, 0xf>(v);  // row_shr:4
  v += dpp_moved<0x118, 0xf>(v);  // row_shr:8
  v += dpp_moved<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_moved<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

template <typename T, int N, bool GATE>
__global__ __launch_bounds__(256, 2) void ssd_kernel(
    const T* __restrict__ x, const T* __restrict__ dt, const float* __restrict__ A_head,
    const T* __restrict__ B, const float4* __restrict__ G, const T* __restrict__ Ct,
    const float* __restrict__ Dskip, const T* __restrict__ z, const float* __restrict__ dt_bias,
    const float* __restrict__ h0, T* __restrict__ y, float* __restrict__ last_state,
    const SsdSizes p) {
  using Op = typename Mma<T>::Op;
  static_assert(sizeof(Op) == sizeof(T), "operands keep the storage type");
  constexpr int Q = 64;            // chunk length
  constexpr int P = 64;            // channels per head
  constexpr int RW = kRunWords<T>;
  constexpr int PADK = 16 / (int)sizeof(Op);   // one 16-byte pad per row
  constexpr int LQ = Q + PADK;     // row length of [.][Q] operand arrays
  // the state index as a product dimension, rounded up to the instruction's K
  // (the staged positions of states N .. KN-1 of the [.][KN] arrays stay zero)
  constexpr int KN = (N + Mma<T>::K - 1) / Mma<T>::K * Mma<T>::K;
  constexpr int PS = Mma<T>::kPackStates;
  constexpr int NPK = (N + PS - 1) / PS;       // state packs (products with H)
  constexpr int TPP = PS / 16;                 // state tiles per pack
  static_assert(KN % PS == 0, "packs cover the staged states");
  constexpr int LN = KN + PADK;    // row length of [.][KN] operand arrays
  constexpr int HT = N / 16;       // state tiles per wave
  constexpr int XI = P * (Q / 8) / 256;        // 8-step runs of x (and z, y) per thread
  constexpr int NR = N * (Q / 8);              // 8-element runs of B (and of B^T, C^T) per chunk
  constexpr int NI = (NR + 255) / 256;         // ... per thread
  static_assert(N % 16 == 0 && N >= 16 && N <= 128, "state count");
  static_assert(P == Q && XI * 256 == P * (Q / 8), "staging layout");

  // Item layouts: 8 consecutive lanes cover one 128-byte piece of a row in
  // global memory and in LDS -- x, z, y runs (p = item / 8, steps
  // 8 * (item % 8)..), B runs (n = item / 8, steps 8 * (item % 8)..) -- and
  // B^T, C^T runs (step item / (N/8), states 8 * (item % (N/8))..) are whole
  // contiguous rows.
  __shared__ __align__(16) Op sX[P][LQ];     // x chunk, [p][t]
  __shared__ __align__(16) Op sXw[P][LQ];    // x o exp(cum_Q - cum_s) Bbar_s, [p][s]
  __shared__ __align__(16) Op sB[N][LQ];     // B chunk, [n][s]
  __shared__ __align__(16) Op sCt[Q][LN];    // C^T, [t][n]
  __shared__ __align__(16) Op sY[P][LQ];     // y in the storage type, [p][t], before its 16-byte stores
  __shared__ __align__(16) Op sM[Q][LQ];     // the masked chunk matrix, [t][s]
  // per step of the chunk: cum2_t = log2 e * sum_{k<=t} Delta_k A and the input
  // coefficient Bbar_t
  __shared__ __align__(16) float sCum2[Q];
  __shared__ __align__(16) float sCoef[Q];
  // Per-step factors, written after the prefix sum and read in step 2 (cum_t
  // as above, c_i = cum_{16i}):
  //   sE0[t]    = exp2(cum_t)                      scales row t of C^T H
  //   sW[s]     = exp2(cum_Q - cum_s) Bbar_s       scales x for the state update
  //   sE1[t]    = exp2(cum_t - c_{t/16})
  //   sW2[i][s] = exp2(c_i - cum_s) Bbar_s, s < 16i
  // so that an off-diagonal mask entry exp2(cum_t - cum_s) Bbar_s (s < 16i <= t)
  // is sE1[t] sW2[i][s]: both factors are partial decays over [s, t], never
  // beyond the entry itself.
  __shared__ __align__(16) float sFac[7 * Q];
  float* const sE0 = sFac;
  float* const sW = sE0 + Q;
  float* const sE1 = sW + Q;
  float(*const sW2)[Q] = reinterpret_cast<float(*)[Q]>(sE1 + Q);  // rows 1..3 used

  // Consecutive block ids go to different XCDs; regroup so that the heads an
  // XCD runs share batch rows (and hence B, C^T and the G tiles in its L2).
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int b = bid / p.nheads;
  const int h = bid % p.nheads;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave: owns channels 16w..
  const int lane = tid & 63;
  const int64_t L = p.seqlen;
  const int dim = p.nheads * P;
  const float Ah = A_head[h];
  const float A2h = Ah * kLog2e;
  const float rAh = 1.0f / Ah;
  const float bias_h = dt_bias != nullptr ? dt_bias[h] : 0.0f;
  const T* xh = x + ((int64_t)b * dim + (int64_t)h * P) * L;
  const T* zh = GATE ? z + ((int64_t)b * dim + (int64_t)h * P) * L : nullptr;
  T* yh = y + ((int64_t)b * dim + (int64_t)h * P) * L;
  const T* Bb = B + (int64_t)b * N * L;
  const int nchunks = (int)((L + Q - 1) / Q);
  const float4* Gb = G + (int64_t)b * nchunks * 10 * 64;
  const T* Ctb = Ct + (int64_t)b * L * N;
  const T* dth = dt + ((int64_t)b * p.nheads + h) * L;

  if constexpr (KN > N) {
    for (int i = tid; i < Q * (KN - N); i += 256)
      sCt[i / (KN - N)][Mma<T>::state_pos(N + i % (KN - N))] = Mma<T>::cvt(0.0f);
  }
  // the two tiles above the diagonal that the diagonal product reads (its K
  // steps of 32 take rows 0..15 up to s < 32 and rows 32..47 up to s < 64)
  // stay zero; the mask step writes only the causal tiles
  for (int i = tid; i < 2 * 16 * 16; i += 256) {
    const int which = i / 256, r = (i % 256) / 16, c = i % 16;
    if (which == 0) sM[r][16 + c] = Mma<T>::cvt(0.0f);
    else sM[32 + r][48 + c] = Mma<T>::cvt(0.0f);
  }

  // the state: wave w owns channels 16w..16w+15, as HT accumulator tiles
  // (states 16k.., channels 16w..)
  f32x4_t H[HT];
#pragma unroll
  for (int k = 0; k < HT; ++k) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = 16 * k + 4 * (lane >> 4) + r, pp = 16 * w + (lane & 15);
      H[k][r] = h0 != nullptr ? h0[((int64_t)b * dim + h * P + pp) * N + n] : 0.0f;
    }
  }
  // Output role: the Y tiles leave the products in accumulator layout, so
  // lane l of wave w holds channel py = 16w + l % 16 and, in t-block i, steps
  // 16i + ty .. +3 (ty = 4 (l / 16)); it forms those y and stages them.
  const int py = 16 * w + (lane & 15);
  const int ty = 4 * (lane >> 4);
  const float Dp = Dskip != nullptr ? Dskip[h * P + py] : 0.0f;

  // A chunk's inputs in registers.  Whole chunks (FULL) take straight vector
  // loads and stores, so the only memory operations in flight across the
  // loop are in program order; the ragged last chunk takes element accesses.
  uint32_t rx[XI][RW], rb[NI][RW], rct[NI][RW];
  uint32_t rz[Q / 16][RW / 2];  // z of the output role's 4 runs of 4 steps
  float4 rg[3];  // this wave's causal tiles of G (wave_mask_tile(w, k))
  T rdt = T(0);  // raw: converted where it is used, so the load is not waited for early
  // whole chunks: buffer accesses with fixed per-lane offsets.  Run item k of
  // x, z, y and B is row tid / 8 + 32k, steps 8 (tid % 8)..; C^T run item k is
  // elements 8 (tid + 256k).. of the chunk's rows.
  constexpr uint32_t ES = sizeof(T);
  const uint32_t vo_run = ((uint32_t)(tid / 8) * (uint32_t)L + 8u * (uint32_t)(tid % 8)) * ES;
  const uint32_t vo_ct = (uint32_t)tid * 8u * ES;
  const uint32_t vo_z = ((uint32_t)py * (uint32_t)L + (uint32_t)ty) * ES;  // z of the output role
  const Buf bufx = make_buf(xh, (int64_t)P * L * ES);
  const Buf bufz = make_buf(GATE ? zh : xh, (int64_t)P * L * ES);
  const Buf bufy = make_buf(yh, (int64_t)P * L * ES);
  const Buf bufB = make_buf(Bb, (int64_t)N * L * ES);
  const Buf bufct = make_buf(Ctb, (int64_t)N * L * ES);
  const Buf bufdt = make_buf(dth, L * ES);
  const Buf bufg = make_buf(Gb, (int64_t)nchunks * 10 * 64 * 16);
  auto row_soff = [&](int k, int64_t c0) { return (uint32_t)((32 * (int64_t)k * L + c0) * ES); };

  // Whole chunks load the next chunk in three parts, each right after this
  // chunk's last use of the registers it fills (spreading the loads over the
  // chunk): B and Delta after step 1, x and C^T after the scaling, the G
  // tiles after the mask.
  auto load_part_b = [&](int64_t c0) {
#pragma unroll
    for (int k = 0; k < NI; ++k)
      if (NR % 256 == 0 || tid + 256 * k < NR) buf_load_run8<T>(bufB, vo_run, row_soff(k, c0), rb[k]);
    buf_load_elem(bufdt, (uint32_t)lane * ES, (uint32_t)(c0 * ES), rdt);
  };
  auto load_part_xc = [&](int64_t c0) {
#pragma unroll
    for (int k = 0; k < XI; ++k) buf_load_run8<T>(bufx, vo_run, row_soff(k, c0), rx[k]);
#pragma unroll
    for (int k = 0; k < NI; ++k)
      if (NR % 256 == 0 || tid + 256 * k < NR)
        buf_load_run8<T>(bufct, vo_ct, (uint32_t)((c0 * N + 2048 * k) * ES), rct[k]);
  };
  auto load_part_g = [&](int64_t c0) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int q = wave_mask_tile(w, k);
      rg[k] = buf_load_f4(bufg, (uint32_t)lane * 16u, (uint32_t)(((c0 / Q) * 10 + (q >= 0 ? q : 9)) * 64 * 16));
    }
  };
  auto load_chunk = [&](auto full_c, int64_t c0) {
    constexpr bool FULL = decltype(full_c)::value;
    if constexpr (FULL) {
      load_part_b(c0);
      load_part_xc(c0);
      load_part_g(c0);
    } else {
      const int tv = (int)(L - c0 < Q ? L - c0 : Q);
#pragma unroll
      for (int k = 0; k < XI; ++k) {
        const int item = tid + 256 * k;
        const int t8 = 8 * (item % 8);
        load_run8<T>(xh + (int64_t)(item / 8) * L + c0 + t8, false, tv - t8, rx[k]);
      }
#pragma unroll
      for (int k = 0; k < NI; ++k) {
        const int item = tid + 256 * k;
        if (NR % 256 == 0 || item < NR) {
          const int t8 = 8 * (item % 8);
          load_run8<T>(Bb + (int64_t)(item / 8) * L + c0 + t8, false, tv - t8, rb[k]);
          const int t = item / (N / 8), n8 = 8 * (item % (N / 8));
          load_run8<T>(Ctb + (c0 + t) * N + n8, t < tv, 0, rct[k]);  // the workspace rows are aligned
        }
      }
      const float4* Gc = Gb + (c0 / Q) * 10 * 64;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int q = wave_mask_tile(w, k);
        rg[k] = Gc[(q >= 0 ? q : 9) * 64 + lane];
      }
      rdt = lane < tv ? dth[c0 + lane] : T(0);
    }
  };
  auto load_gate = [&](auto full_c, int64_t c0) {
    constexpr bool FULL = decltype(full_c)::value;
#pragma unroll
    for (int i = 0; i < Q / 16; ++i) {
      if constexpr (FULL) {
        buf_load_run4<T>(bufz, vo_z, (uint32_t)((c0 + 16 * i) * ES), rz[i]);
      } else {
        float f[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t t = c0 + 16 * i + ty + r;
          f[r] = t < L ? Elem<T>::load(zh + (int64_t)py * L + t) : 0.0f;
        }
        pack_floats<T, 4>(f, rz[i]);
      }
    }
  };

  // One chunk at t0, its inputs (and z) already in registers.  A whole chunk
  // also loads the inputs of the chunk at `next`, and after its output that
  // chunk's z (the last whole chunk reloads its own: the loads stay
  // unconditional).
  auto chunk = [&](auto full_c, int64_t t0, int64_t next) {
    constexpr bool FULL = decltype(full_c)::value;
    const int tvalid = FULL ? Q : (int)(L - t0 < Q ? L - t0 : Q);

    // ---- (1) this chunk's x, B into LDS; Delta, its prefix sum and the per-step factors --
#pragma unroll
    for (int k = 0; k < XI; ++k) {
      const int item = tid + 256 * k;
      lds_store_run<T>(&sX[item / 8][8 * (item % 8)], rx[k]);
    }
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int item = tid + 256 * k;
      if (NR % 256 == 0 || item < NR) {
        lds_store_run<T>(&sB[item / 8][8 * (item % 8)], rb[k]);
      }
    }
    {  // every wave forms the prefix sum (a few DPP steps) and writes its share of the factors
      float dl = 0.0f, coef = 0.0f;
      if (FULL || lane < tvalid) {
        const float xr = raw_value(rdt) + bias_h;
        dl = p.softplus ? softplus_f32(xr) : xr;
        if (p.zoh) {
          const float x2 = dl * A2h;
          coef = zoh_coef(exp2_hw(x2), x2, dl, rAh);
        } else {
          coef = dl;
        }
      }
      const float cum2 = wave_prefix_sum(dl * A2h);
      const float cQ = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum2), Q - 1));
      float cref[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) cref[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum2), 16 * i));
      if (w == 0) {
        sCum2[lane] = cum2;
        sCoef[lane] = coef;
        sE0[lane] = exp2_hw(cum2);
      } else if (w == 1) {
        sW[lane] = exp2_hw(cQ - cum2) * coef;
        sE1[lane] = exp2_hw(cum2 - cref[lane >> 4]);
      } else if (w == 2) {
        sW2[1][lane] = lane < 16 ? exp2_hw(cref[1] - cum2) * coef : 0.0f;
        sW2[2][lane] = lane < 32 ? exp2_hw(cref[2] - cum2) * coef : 0.0f;
      } else {
        sW2[3][lane] = lane < 48 ? exp2_hw(cref[3] - cum2) * coef : 0.0f;
      }
    }
    if constexpr (FULL) load_part_b(next);  // B and Delta are in LDS / used
    __syncthreads();

    // ---- (2) C^T, x o w, the mask (the next chunk's loads in between) ----------------------
    const float cum2Q = sCum2[Q - 1];
    // C^T as loaded (the decay exp2(cum_t) of the state part is applied to
    // the product's rows in step 3)
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int item = tid + 256 * k;
      if (NR % 256 == 0 || item < NR) {
        const int t = item / (N / 8), n8 = 8 * (item % (N / 8));
        lds_store_states<T>(&sCt[t][0], n8, rct[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < XI; ++k) {
      const int item = tid + 256 * k;
      const int pp = item / 8, t8 = 8 * (item % 8);
      const float4 w0 = *reinterpret_cast<const float4*>(&sW[t8]);
      const float4 w1 = *reinterpret_cast<const float4*>(&sW[t8 + 4]);
      const float wvv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = run_elem<T>(rx[k], j) * wvv[j];
      uint32_t wv[RW];
      pack_floats<T, 8>(v, wv);
      lds_store_run<T>(&sXw[pp][t8], wv);
    }
    if constexpr (FULL) load_part_xc(next);  // x and C^T are in LDS

    // the 10 causal 16x16 tiles (t-block i, s-block j <= i) dealt over the 4
    // waves: tile 0 of a wave is its diagonal tile, tiles 1 and 2 (when
    // dealt) lie below the diagonal (wave_mask_tile).  A lane holds 4
    // consecutive s of one t and writes them at once; every LDS read of the
    // wave's tiles is issued before the first is used.
    {
      const int tl = lane & 15, sl = 4 * (lane >> 4);
      const int q1 = wave_mask_tile(w, 1), q2 = wave_mask_tile(w, 2);
      const int i0 = causal_tile_row(wave_mask_tile(w, 0));
      const int i1 = causal_tile_row(q1), j1 = q1 - i1 * (i1 + 1) / 2;
      const bool has2 = q2 >= 0;
      const int i2 = has2 ? causal_tile_row(q2) : 0, j2 = has2 ? q2 - i2 * (i2 + 1) / 2 : 0;
      const int t0d = 16 * i0 + tl, s0d = 16 * i0 + sl;
      const int t1 = 16 * i1 + tl, s01 = 16 * j1 + sl;
      const int t2 = 16 * i2 + tl, s02 = 16 * j2 + sl;
      const float ct = sCum2[t0d];
      const float4 cs = *reinterpret_cast<const float4*>(&sCum2[s0d]);
      const float4 bs = *reinterpret_cast<const float4*>(&sCoef[s0d]);
      const float e1a = sE1[t1];
      const float4 w2a = *reinterpret_cast<const float4*>(&sW2[i1][s01]);
      float e1b = 0.0f;
      float4 w2b = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (has2) {
        e1b = sE1[t2];
        w2b = *reinterpret_cast<const float4*>(&sW2[i2][s02]);
      }
      {  // diagonal tile: the decay between s and t directly
        const float gv[4] = {rg[0].x, rg[0].y, rg[0].z, rg[0].w};
        const float csv[4] = {cs.x, cs.y, cs.z, cs.w}, bsv[4] = {bs.x, bs.y, bs.z, bs.w};
        float mv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) mv[r] = s0d + r <= t0d ? (gv[r] * bsv[r]) * exp2_hw(ct - csv[r]) : 0.0f;
        uint32_t wv[4 * sizeof(T) / 4];
        pack_floats<T, 4>(mv, wv);
        store_words<4 * sizeof(T) / 4>(&sM[t0d][s0d], wv);
      }
      // below the diagonal (s < 16i <= t): the decay split at step 16i
      auto off_tile = [&](const float4& g, float e1, const float4& w2, int t, int s0) {
        float mv[4];
        mv[0] = (g.x * w2.x) * e1;
        mv[1] = (g.y * w2.y) * e1;
        mv[2] = (g.z * w2.z) * e1;
        mv[3] = (g.w * w2.w) * e1;
        uint32_t wv[4 * sizeof(T) / 4];
        pack_floats<T, 4>(mv, wv);
        store_words<4 * sizeof(T) / 4>(&sM[t][s0], wv);
      };
      off_tile(rg[1], e1a, w2a, t1, s01);
      if (has2) off_tile(rg[2], e1b, w2b, t2, s02);
    }
    if constexpr (FULL) load_part_g(next);  // this chunk's G tiles are used
    __syncthreads();

    // ---- (3) Y = M X^T + diag(exp(cum_t)) C^T H for this wave's channels, staged [p][t]
    // ----------------------------------------------------------------------------------
    if constexpr (sizeof(T) == 2) {
      // bf16: every LDS operand of a t-block is read before its first product,
      // so the reads' latencies overlap instead of each product waiting for
      // its own; the x operands of the diagonal product (this wave's channels,
      // both K halves) serve every t-block
      const int rr = lane & 15, kk = 8 * (lane >> 4);
      typename Mma<T>::StatePack hp[NPK];
      const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int m = 0; m < NPK; ++m) {
        const int k1 = TPP * m + 1 < HT ? TPP * m + 1 : HT - 1;
        hp[m] = Mma<T>::pack_state(H[TPP * m], TPP * m + 1 < HT ? H[k1] : zero);
      }
      const bf16x8_t xb0 = lds_frag8(&sX[16 * w + rr][kk]);
      const bf16x8_t xb1 = lds_frag8(&sX[16 * w + rr][32 + kk]);
#pragma unroll
      for (int i = 0; i < Q / 16; ++i) {
        // t-block i needs s < 16 (i + 1): one product of K = 32 for i < 2 (the
        // staged zeros above the diagonal fill it), two for i >= 2
        const bf16x8_t ma0 = lds_frag8(&sM[16 * i + rr][kk]);
        const bf16x8_t ma1 = i >= 2 ? lds_frag8(&sM[16 * i + rr][32 + kk]) : bf16x8_t{};
        bf16x8_t ca[NPK];
#pragma unroll
        for (int m = 0; m < NPK; ++m) ca[m] = lds_frag8(&sCt[16 * i + rr][PS * m + kk]);
        const int tc = 16 * i + ty;
        uint32_t xr[RW / 2];
        load_words<RW / 2>(&sX[py][tc], xr);
        const float4 e4 = *reinterpret_cast<const float4*>(&sE0[tc]);
        f32x4_t yd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ma0, xb0, zero, 0, 0, 0);
        if (i >= 2) yd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ma1, xb1, yd, 0, 0, 0);
        f32x4_t yo = zero;
#pragma unroll
        for (int m = 0; m < NPK; ++m) yo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ca[m], hp[m], yo, 0, 0, 0);
        // y = (Y + D x) silu(z) for this lane's 4 steps, staged in the storage
        // type; the state part takes its decay exp2(cum_t) here
        const float ev[4] = {e4.x, e4.y, e4.z, e4.w};
        float yv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = __builtin_fmaf(Dp, run_elem4<T>(xr, r), __builtin_fmaf(ev[r], yo[r], yd[r]));
          if constexpr (GATE) v *= silu_f32(run_elem4<T>(rz[i], r));
          yv[r] = v;
        }
        uint32_t yw[RW / 2];
        pack_floats<T, 4>(yv, yw);
        store_words<RW / 2>(&sY[py][tc], yw);
      }
      if constexpr (FULL && GATE) load_gate(full_c, next);  // this chunk's z are used
      // H <- exp(cum_Q) H + B (x o w)^T, the B operands of each K half read
      // together before its products
      const float decay = exp2_hw(cum2Q);
#pragma unroll
      for (int k = 0; k < HT; ++k) {
#pragma unroll
        for (int r = 0; r < 4; ++r) H[k][r] *= decay;
      }
#pragma unroll
      for (int k0 = 0; k0 < Q; k0 += 32) {
        const bf16x8_t bx = lds_frag8(&sXw[16 * w + rr][k0 + kk]);
        bf16x8_t ba[HT];
#pragma unroll
        for (int k = 0; k < HT; ++k) ba[k] = lds_frag8(&sB[16 * k + rr][k0 + kk]);
#pragma unroll
        for (int k = 0; k < HT; ++k) H[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ba[k], bx, H[k], 0, 0, 0);
      }
    } else {
      {
        typename Mma<T>::StatePack hp[NPK];
        const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < NPK; ++m) {
          const int k1 = TPP * m + 1 < HT ? TPP * m + 1 : HT - 1;
          hp[m] = Mma<T>::pack_state(H[TPP * m], TPP * m + 1 < HT ? H[k1] : zero);
        }
#pragma unroll
        for (int i = 0; i < Q / 16; ++i) {
          f32x4_t yd = zero, yo = zero;
          // diagonal part: t-block i needs s < 16 (i + 1)
          yd = tile_mma<T>(&sM[0][0], LQ, 16 * i, &sX[0][0], LQ, 16 * w, 16 * (i + 1), lane, yd);
          // the state entering the chunk
#pragma unroll
          for (int m = 0; m < NPK; ++m) yo = Mma<T>::mma_state(&sCt[16 * i][PS * m], LN, hp[m], yo, lane);
          // y = (Y + D x) silu(z) for this lane's 4 steps, staged in the storage type;
          // the state part takes its decay exp2(cum_t) here
          const int tc = 16 * i + ty;
          uint32_t xr[RW / 2];
          load_words<RW / 2>(&sX[py][tc], xr);
          const float4 e4 = *reinterpret_cast<const float4*>(&sE0[tc]);
          const float ev[4] = {e4.x, e4.y, e4.z, e4.w};
          float yv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float v = __builtin_fmaf(Dp, run_elem4<T>(xr, r), __builtin_fmaf(ev[r], yo[r], yd[r]));
            if constexpr (GATE) v *= silu_f32(run_elem4<T>(rz[i], r));
            yv[r] = v;
          }
          uint32_t yw[RW / 2];
          pack_floats<T, 4>(yv, yw);
          store_words<RW / 2>(&sY[py][tc], yw);
        }
      }
      if constexpr (FULL && GATE) load_gate(full_c, next);  // this chunk's z are used
      // ---- H <- exp(cum_Q) H + B (x o w)^T ----------------------------------------------------
      {
        const float decay = exp2_hw(cum2Q);
#pragma unroll
        for (int k = 0; k < HT; ++k) {
#pragma unroll
          for (int r = 0; r < 4; ++r) H[k][r] *= decay;
        }
        const int rr = lane & 15, kk = Mma<T>::KL * (lane >> 4);
#pragma unroll
        for (int k0 = 0; k0 < Q; k0 += Mma<T>::K) {
          const Op* bx = &sXw[16 * w + rr][k0 + kk];
#pragma unroll
          for (int k = 0; k < HT; ++k) H[k] = Mma<T>::mma(&sB[16 * k + rr][k0 + kk], bx, H[k]);
        }
      }
    }
    __syncthreads();

    // ---- (4) the staged y out, 16-byte runs along the rows ------------------------------
#pragma unroll
    for (int k = 0; k < XI; ++k) {
      const int item = tid + 256 * k;
      const int pp = item / 8, t8 = 8 * (item % 8);
      uint32_t yw[RW];
      load_words<RW>(&sY[pp][t8], yw);
      if constexpr (FULL) {
#pragma unroll
        for (int q = 0; q < RW / 4; ++q) {
          const u32x4_t v = {yw[4 * q], yw[4 * q + 1], yw[4 * q + 2], yw[4 * q + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(v, bufy.r, vo_run + 16 * q, row_soff(k, t0), 0);
        }
      } else {
        const int64_t off = (int64_t)pp * L + t0 + t8;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (t8 + j < tvalid) Elem<T>::store(yh + off + j, run_elem<T>(yw, j));
      }
    }
    // no barrier: the next chunk's step 1 writes neither the staging nor
    // anything read here, and its step 3 (which rewrites the staging) comes
    // after two barriers that every wave reaches only past this step
  };

  // whole chunks while the rows allow 16-byte accesses, then the rest
  const int64_t nfull = p.vec ? L / Q : 0;
  if (nfull > 0) {
    load_chunk(BoolC<true>{}, 0);
    if constexpr (GATE) load_gate(BoolC<true>{}, 0);
    // the first chunk is peeled so that the loop is entered with the memory
    // operations of a chunk in flight, as from its own back edge (the
    // compiler's waits at the loop head then count only the loads they need)
    chunk(BoolC<true>{}, 0, (nfull > 1 ? 1 : 0) * Q);
  }
  for (int64_t c = 1; c < nfull; ++c) chunk(BoolC<true>{}, c * Q, (c + 1 < nfull ? c + 1 : c) * Q);
  for (int64_t t0 = nfull * Q; t0 < L; t0 += Q) {
    load_chunk(BoolC<false>{}, t0);
    if constexpr (GATE) load_gate(BoolC<false>{}, t0);
    chunk(BoolC<false>{}, t0, t0);
  }

  if (last_state != nullptr) {
#pragma unroll
    for (int k = 0; k < HT; ++k) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = 16 * k + 4 * (lane >> 4) + r, pp = 16 * w + (lane & 15);
        last_state[((int64_t)b * dim + h * P + pp) * N + n] = H[k][r];
      }
    }
  }
}

template <typename T, int N>
static hipError_t launch_ssd_n(const SsdLaunch& a, hipStream_t stream) {
  SsdSizes s;
  s.batch = a.batch;
  s.nheads = a.nheads;
  s.seqlen = a.seqlen;
  s.softplus = a.softplus;
  s.zoh = a.zoh;
  s.vec = a.vec;
  const int nchunks = (int)((a.seqlen + 63) / 64);
  T* Ct = static_cast<T*>(a.ws);
  float4* G = reinterpret_cast<float4*>(static_cast<char*>(a.ws) +
                                        ssd_ws_ct_bytes(a.batch, N, a.seqlen, (int)sizeof(T)));
  ssd_prep_kernel<T, N><<<(unsigned)(a.batch * nchunks), 256, 0, stream>>>(
      static_cast<const T*>(a.B), static_cast<const T*>(a.C), Ct, G, a.seqlen, nchunks, a.vec);
  auto kernel = a.z != nullptr ? ssd_kernel<T, N, true> : ssd_kernel<T, N, false>;
  kernel<<<(unsigned)(a.batch * a.nheads), 256, 0, stream>>>(
      static_cast<const T*>(a.x), static_cast<const T*>(a.dt), a.A, static_cast<const T*>(a.B), G,
      Ct, a.Dskip, static_cast<const T*>(a.z), a.dt_bias, a.h0, static_cast<T*>(a.y),
      a.last_state, s);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_ssd_t(const SsdLaunch& a, hipStream_t stream) {
  switch (a.dstate) {
    case 16: return launch_ssd_n<T, 16>(a, stream);
    case 32: return launch_ssd_n<T, 32>(a, stream);
    case 64: return launch_ssd_n<T, 64>(a, stream);
    case 128:
      if constexpr (sizeof(T) == 2) return launch_ssd_n<T, 128>(a, stream);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_ssd_fwd(const SsdLaunch& a, hipStream_t stream) {
  if (a.batch == 0 || a.nheads == 0 || a.seqlen == 0) return hipSuccess;
  if (a.headdim != kSsdHeadDim) return hipErrorInvalidValue;
  return a.dtype == Dtype::BF16 ? launch_ssd_t<uint16_t>(a, stream) : launch_ssd_t<float>(a, stream);
}

}  // namespace ssm
