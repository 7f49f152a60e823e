// ssm_kernels.hpp -- host-side launch interface between the C ABI layer
// (ssm_api.cpp) and the HIP kernels (scan_fwd.hip, state_update.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

// Time steps one workgroup stages per tile of the forward scan.
constexpr int kScanTile = 16;

// Tiles of the forward scan whose u/delta/z loads are issued together (a
// load block): enough to cover a 128-byte line of every row, so each line is
// fetched once rather than once per tile, within a budget of 8 32-bit words
// of each array per thread.  A thread loads TL/G steps of a tile.
constexpr int scan_load_block_tiles(int elem_bytes, int G, int TL = kScanTile) {
  const int W = (TL / G) * elem_bytes / 4;
  const int by_line = 128 / (TL * elem_bytes);
  const int by_regs = 8 / W;
  const int kt = by_line < by_regs ? by_line : by_regs;
  return kt < 1 ? 1 : (kt > 4 ? 4 : kt);
}

// Storage type of the per-token tensors.
enum class Dtype { F32 = 0, BF16 = 1 };

// Passes of the forward scan kernel (its PASS template argument).
constexpr int kPassMain = 0;  // y and last_state
constexpr int kPassAgg = 1;   // segment aggregates (end state from zero, Delta sum)
constexpr int kPassCkpt = 2;  // the state entering every tile, for the backward pass
constexpr int kPassMainCkpt = 3;  // y and last_state, and the state entering every tile

// Kernel variants (bits of the MODE template argument).
constexpr int kModeZoh = 1;   // zero-order-hold input term (else Euler)
constexpr int kModeConv = 2;  // causal depthwise conv1d + silu applied to the input first

struct ScanLaunch {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;     // nullable
  const void* z;          // nullable
  const float* bias;      // nullable
  const float* h0;        // nullable
  void* y;
  float* last_state;      // nullable
  void* ws_bc;            // (batch, G, seqlen, 2*dstate/G) B, C records, input type
  float* ws_hend;         // (nseg-1, batch, dim, dstate) when nseg > 1
  float* ws_sumdt;        // (nseg-1, batch, dim) when nseg > 1
  int batch, dim, dstate;
  int64_t seqlen;
  int64_t seglen;         // multiple of kScanTile
  int nseg;               // segments the sequence is split into
  int softplus;
  int vec;                // 16-byte vector loads/stores allowed
  int vec_bc;             // B and C rows 16-byte aligned (time-parallel kernel)
  int ncu;                // compute units of the device
  int prio_blocks;        // load blocks per wave-priority step (0: no rotation)
  int zoh;                // zero-order-hold input term (else Euler)
  // convolution prologue (conv_w null: none); u then holds its input x
  const float* conv_w;          // (dim, conv_k)
  const float* conv_b;          // (dim) nullable
  const float* conv_state_in;   // (batch, dim, conv_k-1) nullable
  float* conv_state_out;        // (batch, dim, conv_k-1) nullable
  int conv_k;                   // 1..4
  // checkpoints, the state entering every tile: (batch, ntiles, N, dim).  With
  // ckpt_with_y the main pass writes them beside y (a forward pass whose
  // backward follows); otherwise a checkpoint pass replaces the main pass.
  float* ws_ckpt;
  int ckpt_with_y;
  Dtype dtype;
};

struct DecodeLaunch {
  float* state;
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;     // nullable
  const void* z;          // nullable
  const float* bias;      // nullable
  void* y;
  int batch, dim, dstate;
  int softplus;
  int vec;                // state and A 16-byte aligned, B and C aligned to 4 elements
  int zoh;                // zero-order-hold input term (else Euler)
  // convolution prologue (conv_w null: none); u then holds the token's x
  float* conv_state;      // (batch, dim, conv_k-1), shifted in place; null when conv_k == 1
  const float* conv_w;    // (dim, conv_k)
  const float* conv_b;    // (dim) nullable
  int conv_k;             // 1..4
  Dtype dtype;
};

// Widest convolution the kernels take.
constexpr int kMaxConvWidth = 4;

// Backward pass (either input term, no convolution prologue).  The caller has
// already put the checkpoints in ws_ckpt and the B, C records in ws_bc: by the
// forward checkpoint pass (launch_scan_fwd with ws_ckpt, which packs the
// records too), or by a forward pass that wrote the checkpoints beside y,
// followed by launch_pack_records.
struct BwdLaunch {
  int zoh;                // zero-order-hold input term (else Euler)
  const void* u;
  const void* delta;
  const float* A;
  const float* Dskip;     // nullable
  const void* z;          // nullable
  const float* bias;      // nullable
  const void* dy;
  const float* dlast;     // nullable
  void* du;
  void* ddelta;
  void* dz;               // required when z is given
  float* dh0;             // nullable
  float* dA;
  void* dB;
  void* dC;
  float* dD;              // nullable
  float* dbias;           // nullable
  const void* ws_bc;      // B, C records (batch, G, seqlen, 2*dstate/G)
  const float* ws_ckpt;   // (batch, ntiles, dstate, dim)
  float* ws_lagg;         // (nseg-1, batch, dim, dstate) when nseg > 1
  float* ws_lsum;         // (nseg-1, batch, dim) when nseg > 1
  float* ws_part_bc;      // (batch, ncg, 2, dstate, seqlen)
  float* ws_part_a;       // (batch, nseg, dim, dstate)
  float* ws_part_d;       // (batch, nseg, dim)
  float* ws_part_bias;    // (batch, nseg, dim)
  int batch, dim, dstate;
  int64_t seqlen, seglen;
  int nseg;
  int softplus;
  int vec;
  Dtype dtype;
};

// SSD (scalar A per head) forward: heads of kSsdHeadDim channels.
constexpr int kSsdHeadDim = 64;
// The SSD workspace: C^T, (batch, seqlen, dstate) in the input type, padded
// to 256 bytes, then per (batch row, 64-step chunk) the 10 causal 16x16 tiles
// of C^T B in float32.
inline size_t ssd_ws_ct_bytes(int batch, int dstate, int64_t seqlen, int elem_bytes) {
  const size_t ct = (size_t)batch * (size_t)seqlen * (size_t)dstate * (size_t)elem_bytes;
  return (ct + 255) / 256 * 256;
}
inline size_t ssd_ws_bytes(int batch, int dstate, int64_t seqlen, int elem_bytes) {
  const size_t nchunks = (size_t)((seqlen + 63) / 64);
  return ssd_ws_ct_bytes(batch, dstate, seqlen, elem_bytes) + (size_t)batch * nchunks * 10 * 256 * 4;
}

struct SsdLaunch {
  const void* x;          // (batch, nheads * headdim, seqlen)
  const void* dt;         // (batch, nheads, seqlen), raw (bias, softplus applied inside)
  const float* A;         // (nheads)
  const void* B;          // (batch, dstate, seqlen), shared by the heads
  const void* C;
  const float* Dskip;     // (nheads * headdim) nullable
  const void* z;          // nullable
  const float* dt_bias;   // (nheads) nullable
  const float* h0;        // (batch, nheads * headdim, dstate) nullable
  void* y;
  float* last_state;      // nullable
  void* ws;               // C^T (batch, seqlen, dstate), input type; then the G tiles
  int batch, nheads, headdim, dstate;
  int64_t seqlen;
  int softplus, zoh, vec;
  Dtype dtype;
};

hipError_t launch_scan_fwd(const ScanLaunch& a, hipStream_t stream);
// Packs only the B, C records into a.ws_bc (a backward pass whose checkpoints
// came from the forward pass needs them and nothing else of launch_scan_fwd).
hipError_t launch_pack_records(const ScanLaunch& a, hipStream_t stream);
// The time-parallel forward scan for long sequences with few channels
// (scan_wave.hip): N = 16, no convolution prologue, no checkpoints; it reads
// B and C directly and needs no workspace.
hipError_t launch_scan_wave(const ScanLaunch& a, hipStream_t stream);
hipError_t launch_ssd_fwd(const SsdLaunch& a, hipStream_t stream);
hipError_t launch_scan_bwd(const BwdLaunch& a, hipStream_t stream);
hipError_t launch_state_update(const DecodeLaunch& a, hipStream_t stream);
// last_state = h0 (or zeros when h0 is null) for an empty sequence.
hipError_t launch_fill_state(float* dst, const float* src, int64_t n, hipStream_t stream);

}  // namespace ssm
