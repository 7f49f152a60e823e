// ssm_api.cpp -- the C ABI of libssm (declared in include/ssm.h): argument
// validation, choice of the launch plan, and the calls into the kernels.
//
// Every check happens before the first HIP call, so a rejected call enqueues
// nothing and the validation can be exercised without a GPU.
#include <atomic>
#include <climits>
#include <cstdint>
#include <cstdlib>

#include "ssm.h"
#include "ssm_kernels.hpp"

namespace {

using ssm::Dtype;

// The forward scan's workgroups are sized so that five fit on a CU (20
// waves); the planner splits a sequence into segments only as far as needed
// to give each of the 256 CUs of an MI355X (gfx950) its five workgroups, and
// never into segments shorter than kMinSegment steps unless forced.
constexpr int64_t kPlanCUs = 256;
constexpr int64_t kWavesPerCU = 20;
constexpr int64_t kMinSegment = 256;

struct SegPlan {
  int nseg;
  int64_t seglen;
};

// Compute units of the current device, cached per device ordinal.
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Load blocks per step of the wave-priority rotation of the forward scan
// (SSM_SCAN_PRIO_BLOCKS overrides; 0 switches the rotation off).  A step
// every block measured fastest (c3 0.582 -> 0.564 ms against eight steps per
// segment; one every tile was slower again).
int prio_blocks() {
  if (const char* env = std::getenv("SSM_SCAN_PRIO_BLOCKS")) {
    const int v = std::atoi(env);
    if (v >= 0) return v;
  }
  return 1;
}

// Whether the forward scan runs on the time-parallel kernel (scan_wave.hip)
// instead of the channel-parallel one.  Only SSM_SCAN_WAVE=1 selects it,
// wherever it applies (16 states, no convolution prologue): on the long
// sequences it was written for it measured slower than the segment split
// (batch 1, D 2048, L 65536, bf16: 1.17 against 0.84 ms), so it is kept for
// comparison, not chosen by the plan.
bool use_wave_kernel(int dstate, bool conv) {
  if (dstate != 16 || conv) return false;
  const char* env = std::getenv("SSM_SCAN_WAVE");
  return env != nullptr && std::atoi(env) != 0;
}

bool dstate_ok(int n) { return n == 1 || n == 2 || n == 4 || n == 8 || n == 16; }

int elem_bytes(int dtype) { return dtype == SSM_BF16 ? 2 : 4; }

bool flags_ok(int flags) { return (flags & ~(SSM_DELTA_SOFTPLUS | SSM_BBAR_ZOH)) == 0; }

// Segments of the sequence for the forward scan.  A chosen segment length is
// a whole number of the kernel's load blocks, so that every block of every
// segment but the last is whole (its lines loaded and stored whole).
// SSM_SCAN_SEGMENTS (an integer >= 1) overrides the choice, with segments of
// whole tiles only; tests use it to run the carry path at small sizes and at
// segment starts inside a load block.
SegPlan plan_segments(int batch, int dim, int dstate, int64_t L, int dtype) {
  const int64_t tile = ssm::kScanTile;
  const int64_t G = dstate >= 4 ? dstate / 4 : 1;
  const int64_t ncg = (dim + 63) / 64;
  const int64_t groups = (int64_t)batch * ncg;        // workgroups per segment
  const int64_t capacity = kPlanCUs * kWavesPerCU / G;  // resident workgroups
  int64_t want = groups > 0 ? capacity / groups : 1;
  int64_t cap = L / kMinSegment;
  int64_t granule = tile * ssm::scan_load_block_tiles(elem_bytes(dtype), (int)G);
  if (const char* env = std::getenv("SSM_SCAN_SEGMENTS")) {
    const long long v = std::atoll(env);
    if (v >= 1) {
      want = v;
      cap = want;
      granule = tile;
    }
  }
  if (want > cap) want = cap;
  const int64_t tiles = (L + tile - 1) / tile;
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  int64_t seglen = (L + want - 1) / want;
  seglen = (seglen + granule - 1) / granule * granule;
  if (seglen < tile) seglen = tile;
  const int64_t nseg = (L + seglen - 1) / seglen;
  return SegPlan{(int)(nseg < 1 ? 1 : nseg), seglen};
}

// Workspace: the B, C records in the input type (always), then for a split sequence the
// end state and Delta sum of every segment but the last; each part 256-byte
// aligned.
struct WsLayout {
  size_t bc, hend, sumdt, total;
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

WsLayout workspace_layout(int batch, int dim, int dstate, int64_t L, int dtype, const SegPlan& sp) {
  WsLayout w{};
  const size_t plane = (size_t)batch * (size_t)dim;
  w.bc = 0;
  w.hend = round256((size_t)batch * (size_t)L * 2 * (size_t)dstate * (size_t)elem_bytes(dtype));
  size_t end = w.hend;
  if (sp.nseg > 1) {
    w.sumdt = w.hend + round256((size_t)(sp.nseg - 1) * plane * (size_t)dstate * sizeof(float));
    end = w.sumdt + round256((size_t)(sp.nseg - 1) * plane * sizeof(float));
  } else {
    w.sumdt = end;
  }
  w.total = end;
  return w;
}

// Backward workspace: the forward layout first (records, segment aggregates),
// then the tile checkpoints, the reverse aggregates and the partial sums.
struct BwdWsLayout {
  WsLayout fwd;
  size_t ckpt, lagg, lsum, part_bc, part_a, part_d, part_bias, total;
};

// Bytes of the tile checkpoints: the state entering every kScanTile-step tile,
// (batch, ntiles, dstate, dim) float32.
size_t ckpt_bytes_of(int batch, int dim, int dstate, int64_t L) {
  const size_t ntiles = (size_t)((L + ssm::kScanTile - 1) / ssm::kScanTile);
  return (size_t)batch * ntiles * (size_t)dstate * (size_t)dim * sizeof(float);
}

// with_ckpt false: the checkpoints come from the caller (the forward pass
// wrote them), so the workspace holds no region for them.
BwdWsLayout bwd_workspace_layout(int batch, int dim, int dstate, int64_t L, int dtype, const SegPlan& sp,
                                 bool with_ckpt = true) {
  BwdWsLayout w{};
  w.fwd = workspace_layout(batch, dim, dstate, L, dtype, sp);
  const size_t plane = (size_t)batch * (size_t)dim;
  const size_t ncg = (size_t)((dim + 63) / 64);
  const size_t segs = (size_t)sp.nseg;
  size_t off = round256(w.fwd.total);
  w.ckpt = off;
  if (with_ckpt) off += round256(ckpt_bytes_of(batch, dim, dstate, L));
  w.lagg = off;
  off += round256((segs - 1) * plane * (size_t)dstate * sizeof(float));
  w.lsum = off;
  off += round256((segs - 1) * plane * sizeof(float));
  w.part_bc = off;
  off += round256((size_t)batch * ncg * 2 * (size_t)dstate * (size_t)L * sizeof(float));
  w.part_a = off;
  off += round256((size_t)batch * segs * (size_t)dim * (size_t)dstate * sizeof(float));
  w.part_d = off;
  off += round256((size_t)batch * segs * (size_t)dim * sizeof(float));
  w.part_bias = off;
  off += round256((size_t)batch * segs * (size_t)dim * sizeof(float));
  w.total = off;
  return w;
}

bool aligned(const void* p, size_t a) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The byte range [lo, hi) a buffer occupies; a null pointer or zero bytes
// occupies none.  Aliasing is judged on these ranges, not on pointer
// equality, so an output that starts inside an input (or ends inside one) is
// rejected too.
struct Span {
  uintptr_t lo, hi;
};

Span span(const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  if (p == nullptr || bytes == 0) return Span{0, 0};
  return Span{lo, lo + bytes};
}

bool overlap(const Span& a, const Span& b) {
  return a.hi > a.lo && b.hi > b.lo && a.lo < b.hi && b.lo < a.hi;
}

// Whether a buffer the call writes overlaps another buffer the call writes,
// or one it reads.  Inputs may overlap each other (they are only read).
template <size_t NO, size_t NI>
bool writes_overlap(const Span (&outs)[NO], const Span (&ins)[NI]) {
  for (size_t i = 0; i < NO; ++i) {
    for (size_t j = i + 1; j < NO; ++j)
      if (overlap(outs[i], outs[j])) return true;
    for (size_t j = 0; j < NI; ++j)
      if (overlap(outs[i], ins[j])) return true;
  }
  return false;
}

// The scan kernels' vectorised paths address the rows of a 64-channel group
// through buffer descriptors with a 32-bit per-lane offset (channel * L +
// step) * element bytes.  Every lane of the group forms one, also the lanes
// past dim (whose accesses fall beyond the descriptor's extent and are
// dropped), so 64 rows must span less than 2^31 bytes whatever dim is:
// sequences of up to 16M bf16 or 8M float32 steps.  Longer ones take the
// element-wise path.
bool group_rows_fit(int64_t seqlen, size_t es) {
  return (long double)64 * (long double)seqlen * (long double)es < (long double)INT32_MAX;
}

// The scan kernels keep step positions in 32 bits.
constexpr int64_t kMaxSeqlen = INT32_MAX - 4096;

bool shapes_fit(int batch, int dim, int64_t seqlen) {
  if (batch < 0 || dim < 0 || seqlen < 0 || seqlen > kMaxSeqlen) return false;
  const long double total = (long double)batch * (long double)dim * (long double)(seqlen > 0 ? seqlen : 1);
  return total < (long double)(INT64_C(1) << 60);
}

}  // namespace

extern "C" {

size_t ssm_scan_fwd_workspace_bytes(int batch, int dim, int dstate, int64_t seqlen, int dtype) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return 0;
  if (!dstate_ok(dstate) || !shapes_fit(batch, dim, seqlen)) return 0;
  if (batch == 0 || dim == 0 || seqlen == 0) return 0;
  return workspace_layout(batch, dim, dstate, seqlen, dtype, plan_segments(batch, dim, dstate, seqlen, dtype))
      .total;
}

}  // extern "C"

namespace {

// ---- scratch of the allocation-free entry point ------------------------------
// ssm_scan_fwd_noalloc keeps its workspace (the B, C records and the segment
// aggregates) in this file-scope device array instead of a caller's buffer.
// Each device holds its own copy, at its own address, from the time the
// library's code object is loaded on it until the process ends.  In host code
// `scratch` only stands in for the symbol: its device address comes from
// hipGetSymbolAddress, once per device (with that device current), and only
// that address is ever passed to a kernel.
constexpr size_t kNoAllocScratchBytes = SSM_NOALLOC_SCRATCH_BYTES;
constexpr int kStatusScratch = SSM_ERR_SCRATCH;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

void* noalloc_scratch() {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> ptrs[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
  ptrs[dev].store(q, std::memory_order_release);
  return q;
}

// Operands of the convolution prologue (all null / zero: no convolution).
struct ConvIn {
  const float* w;
  const float* b;
  const float* state_in;   // scan only
  float* state_out;        // scan only
  float* state;            // decode only, in place
  int k;
};

bool conv_aligned(const ConvIn* cv) {
  return cv == nullptr || (aligned(cv->w, 4) && aligned(cv->b, 4) && aligned(cv->state_in, 4) &&
                           aligned(cv->state_out, 4) && aligned(cv->state, 4));
}

int scan_impl(const void* u, const void* delta, const float* A, const void* B, const void* C,
              const float* D_skip, const void* z, const float* delta_bias, int flags,
              const float* h0, void* y, float* last_state, int batch, int dim, int dstate,
              int64_t seqlen, int dtype, void* workspace, size_t workspace_bytes, void* stream,
              const ConvIn* cv, bool use_scratch = false, bool want_ckpt = false,
              float* ckpt = nullptr, size_t ckpt_bytes = 0) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (!flags_ok(flags)) return SSM_ERR_FLAGS;
  if (!dstate_ok(dstate) || !shapes_fit(batch, dim, seqlen)) return SSM_ERR_SHAPE;
  if (cv != nullptr && (cv->k < 1 || cv->k > ssm::kMaxConvWidth)) return SSM_ERR_SHAPE;
  const bool empty = batch == 0 || dim == 0;
  if (!empty && seqlen > 0 && (!u || !delta || !A || !B || !C || !y)) return SSM_ERR_NULL;
  if (!empty && cv != nullptr && cv->w == nullptr) return SSM_ERR_NULL;
  const size_t es = (size_t)elem_bytes(dtype);
  if (!aligned(u, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) ||
      !aligned(z, es) || !aligned(y, es) || !aligned(A, 4) || !aligned(D_skip, 4) ||
      !aligned(delta_bias, 4) || !aligned(h0, 4) || !aligned(last_state, 4) ||
      !aligned(workspace, 256) || !aligned(ckpt, 4))
    return SSM_ERR_ALIGN;
  if (!conv_aligned(cv)) return SSM_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (empty) return SSM_OK;
  // the checkpoints: every tile's entering state, so none for an empty sequence
  const size_t ckb = want_ckpt ? ckpt_bytes_of(batch, dim, dstate, seqlen) : 0;
  if (ckb > 0 && ckpt == nullptr) return SSM_ERR_NULL;
  if (ckb > 0 && ckpt_bytes < ckb) return SSM_ERR_WORKSPACE;
  {
    const size_t tok = (size_t)batch * (size_t)dim * (size_t)seqlen * es;
    const size_t bc = (size_t)batch * (size_t)dstate * (size_t)seqlen * es;
    const size_t per_dim = (size_t)dim * sizeof(float);
    const size_t state = (size_t)batch * (size_t)dim * (size_t)dstate * sizeof(float);
    const size_t ck = cv != nullptr && cv->k > 1 ? (size_t)batch * (size_t)dim * (size_t)(cv->k - 1) * 4 : 0;
    const size_t cw = cv != nullptr ? (size_t)dim * (size_t)cv->k * 4 : 0;
    const Span outs[] = {span(y, tok), span(last_state, state),
                         span(cv != nullptr ? cv->state_out : nullptr, ck), span(ckpt, ckb)};
    const Span ins[] = {span(u, tok), span(delta, tok), span(z, tok), span(B, bc), span(C, bc),
                        span(A, per_dim * (size_t)dstate), span(D_skip, per_dim),
                        span(delta_bias, per_dim), span(h0, state),
                        span(cv != nullptr ? cv->w : nullptr, cw),
                        span(cv != nullptr ? cv->b : nullptr, cv != nullptr ? per_dim : 0),
                        span(cv != nullptr ? cv->state_in : nullptr, ck)};
    if (writes_overlap(outs, ins)) return SSM_ERR_ALIAS;
  }

  if (seqlen == 0) {  // nothing to scan: the states stay as they came in (or zero)
    if (last_state != nullptr) {
      const hipError_t e = ssm::launch_fill_state(last_state, h0, (int64_t)batch * dim * dstate, st);
      if (e != hipSuccess) return SSM_ERR_HIP;
    }
    if (cv != nullptr && cv->state_out != nullptr && cv->k > 1) {
      const hipError_t e =
          ssm::launch_fill_state(cv->state_out, cv->state_in, (int64_t)batch * dim * (cv->k - 1), st);
      if (e != hipSuccess) return SSM_ERR_HIP;
    }
    return SSM_OK;
  }

  const SegPlan sp = plan_segments(batch, dim, dstate, seqlen, dtype);
  const int64_t blocks = (int64_t)batch * ((dim + 63) / 64) * sp.nseg;
  const int64_t pack_blocks = (int64_t)batch * ((seqlen + 255) / 256);
  if (blocks > INT_MAX || pack_blocks > INT_MAX) return SSM_ERR_SHAPE;
  const WsLayout wl = workspace_layout(batch, dim, dstate, seqlen, dtype, sp);
  if (use_scratch) {
    // every argument is valid by now: the first HIP call is the symbol lookup
    if (wl.total > kNoAllocScratchBytes) return kStatusScratch;
    workspace = noalloc_scratch();
    if (workspace == nullptr) return SSM_ERR_HIP;
    workspace_bytes = kNoAllocScratchBytes;
  }
  if (workspace == nullptr || workspace_bytes < wl.total) return SSM_ERR_WORKSPACE;
  {
    const size_t tok = (size_t)batch * (size_t)dim * (size_t)seqlen * es;
    const size_t bc = (size_t)batch * (size_t)dstate * (size_t)seqlen * es;
    const size_t state = (size_t)batch * (size_t)dim * (size_t)dstate * sizeof(float);
    const size_t ck = cv != nullptr && cv->k > 1 ? (size_t)batch * (size_t)dim * (size_t)(cv->k - 1) * 4 : 0;
    const Span outs[] = {span(workspace, wl.total)};
    const Span ins[] = {span(u, tok), span(delta, tok), span(z, tok), span(B, bc), span(C, bc),
                        span(A, (size_t)dim * (size_t)dstate * 4), span(D_skip, (size_t)dim * 4),
                        span(delta_bias, (size_t)dim * 4), span(h0, state), span(y, tok),
                        span(last_state, state),
                        span(cv != nullptr ? cv->w : nullptr, cv != nullptr ? (size_t)dim * (size_t)cv->k * 4 : 0),
                        span(cv != nullptr ? cv->b : nullptr, cv != nullptr ? (size_t)dim * 4 : 0),
                        span(cv != nullptr ? cv->state_in : nullptr, ck),
                        span(cv != nullptr ? cv->state_out : nullptr, ck), span(ckpt, ckb)};
    if (writes_overlap(outs, ins)) return SSM_ERR_ALIAS;
  }

  ssm::ScanLaunch a{};
  a.u = u;
  a.delta = delta;
  a.A = A;
  a.B = B;
  a.C = C;
  a.Dskip = D_skip;
  a.z = z;
  a.bias = delta_bias;
  a.h0 = h0;
  a.y = y;
  a.last_state = last_state;
  char* ws = static_cast<char*>(workspace);
  a.ws_bc = ws + wl.bc;
  if (sp.nseg > 1) {
    a.ws_hend = reinterpret_cast<float*>(ws + wl.hend);
    a.ws_sumdt = reinterpret_cast<float*>(ws + wl.sumdt);
  }
  a.batch = batch;
  a.dim = dim;
  a.dstate = dstate;
  a.seqlen = seqlen;
  a.seglen = sp.seglen;
  a.nseg = sp.nseg;
  a.softplus = (flags & SSM_DELTA_SOFTPLUS) ? 1 : 0;
  a.zoh = (flags & SSM_BBAR_ZOH) ? 1 : 0;
  if (cv != nullptr) {
    a.conv_w = cv->w;
    a.conv_b = cv->b;
    a.conv_state_in = cv->state_in;
    a.conv_state_out = cv->state_out;
    a.conv_k = cv->k;
  }
  const bool rows16 = ((int64_t)es * seqlen) % 16 == 0;
  a.vec = rows16 && group_rows_fit(seqlen, es) && aligned(u, 16) && aligned(delta, 16) &&
          aligned(z, 16) && aligned(y, 16);
  a.vec_bc = rows16 && aligned(B, 16) && aligned(C, 16);
  a.dtype = dtype == SSM_BF16 ? Dtype::BF16 : Dtype::F32;
  a.ncu = device_cu_count();
  a.prio_blocks = prio_blocks();
  if (ckb > 0) {
    a.ws_ckpt = ckpt;
    a.ckpt_with_y = 1;
    return ssm::launch_scan_fwd(a, st) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
  }
  if (use_wave_kernel(dstate, cv != nullptr))
    return ssm::launch_scan_wave(a, st) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
  return ssm::launch_scan_fwd(a, st) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int update_impl(float* state, const void* u, const void* delta, const float* A, const void* B,
                const void* C, const float* D_skip, const void* z, const float* delta_bias,
                int flags, void* y, int batch, int dim, int dstate, int dtype, void* stream,
                const ConvIn* cv) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (!flags_ok(flags)) return SSM_ERR_FLAGS;
  if (!dstate_ok(dstate) || !shapes_fit(batch, dim, 1)) return SSM_ERR_SHAPE;
  if (cv != nullptr && (cv->k < 1 || cv->k > ssm::kMaxConvWidth)) return SSM_ERR_SHAPE;
  const bool empty = batch == 0 || dim == 0;
  if (!empty && (!state || !u || !delta || !A || !B || !C || !y)) return SSM_ERR_NULL;
  if (!empty && cv != nullptr && (cv->w == nullptr || (cv->k > 1 && cv->state == nullptr)))
    return SSM_ERR_NULL;
  const size_t es = (size_t)elem_bytes(dtype);
  if (!aligned(state, 4) || !aligned(u, es) || !aligned(delta, es) || !aligned(B, es) ||
      !aligned(C, es) || !aligned(z, es) || !aligned(y, es) || !aligned(A, 4) ||
      !aligned(D_skip, 4) || !aligned(delta_bias, 4))
    return SSM_ERR_ALIGN;
  if (!conv_aligned(cv)) return SSM_ERR_ALIGN;
  if (empty) return SSM_OK;
  {
    const size_t tok = (size_t)batch * (size_t)dim * es;
    const size_t bc = (size_t)batch * (size_t)dstate * es;
    const size_t per_dim = (size_t)dim * sizeof(float);
    const size_t ck = cv != nullptr && cv->k > 1 ? (size_t)batch * (size_t)dim * (size_t)(cv->k - 1) * 4 : 0;
    // the state and the carried convolution inputs are read and written in place
    const Span outs[] = {span(y, tok), span(state, (size_t)batch * (size_t)dim * (size_t)dstate * 4),
                         span(cv != nullptr ? cv->state : nullptr, ck)};
    const Span ins[] = {span(u, tok), span(delta, tok), span(z, tok), span(B, bc), span(C, bc),
                        span(A, per_dim * (size_t)dstate), span(D_skip, per_dim),
                        span(delta_bias, per_dim),
                        span(cv != nullptr ? cv->w : nullptr, cv != nullptr ? per_dim * (size_t)cv->k : 0),
                        span(cv != nullptr ? cv->b : nullptr, cv != nullptr ? per_dim : 0)};
    if (writes_overlap(outs, ins)) return SSM_ERR_ALIAS;
  }
  // one grid row per batch row: its lanes (P per channel) are indexed in 32 bits
  if ((int64_t)dim * (dstate >= 4 ? dstate / 4 : 1) + 255 > INT_MAX) return SSM_ERR_SHAPE;

  ssm::DecodeLaunch a{};
  a.state = state;
  a.u = u;
  a.delta = delta;
  a.A = A;
  a.B = B;
  a.C = C;
  a.Dskip = D_skip;
  a.z = z;
  a.bias = delta_bias;
  a.y = y;
  a.batch = batch;
  a.dim = dim;
  a.dstate = dstate;
  a.softplus = (flags & SSM_DELTA_SOFTPLUS) ? 1 : 0;
  a.zoh = (flags & SSM_BBAR_ZOH) ? 1 : 0;
  if (cv != nullptr) {
    a.conv_state = cv->state;
    a.conv_w = cv->w;
    a.conv_b = cv->b;
    a.conv_k = cv->k;
  }
  // vector path: 16-byte state, A rows and (per lane) B, C pieces
  a.vec = (aligned(state, 16) && aligned(A, 16) && aligned(B, 4 * es) && aligned(C, 4 * es)) ? 1 : 0;
  a.dtype = dtype == SSM_BF16 ? Dtype::BF16 : Dtype::F32;
  return ssm::launch_state_update(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SSM_OK
                                                                                    : SSM_ERR_HIP;
}

}  // namespace

extern "C" {

int ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                 const float* D_skip, const void* z, const float* delta_bias, int flags,
                 const float* h0, void* y, float* last_state, int batch, int dim, int dstate,
                 int64_t seqlen, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
  return scan_impl(u, delta, A, B, C, D_skip, z, delta_bias, flags, h0, y, last_state, batch, dim,
                   dstate, seqlen, dtype, workspace, workspace_bytes, stream, nullptr);
}

int ssm_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B,
                         const void* C, const float* D_skip, const void* z, const float* delta_bias,
                         int flags, const float* h0, void* y, float* last_state, int batch, int dim,
                         int dstate, int64_t seqlen, int dtype, void* stream) {
  return scan_impl(u, delta, A, B, C, D_skip, z, delta_bias, flags, h0, y, last_state, batch, dim,
                   dstate, seqlen, dtype, nullptr, 0, stream, nullptr, true);
}

int ssm_conv_scan_fwd(const void* x, const float* conv_w, const float* conv_b, int conv_width,
                      const float* conv_state_in, float* conv_state_out, const void* delta,
                      const float* A, const void* B, const void* C, const float* D_skip,
                      const void* z, const float* delta_bias, int flags, const float* h0, void* y,
                      float* last_state, int batch, int dim, int dstate, int64_t seqlen, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const ConvIn cv{conv_w, conv_b, conv_state_in, conv_state_out, nullptr, conv_width};
  return scan_impl(x, delta, A, B, C, D_skip, z, delta_bias, flags, h0, y, last_state, batch, dim,
                   dstate, seqlen, dtype, workspace, workspace_bytes, stream, &cv);
}

int ssm_state_update(float* state, const void* u, const void* delta, const float* A,
                     const void* B, const void* C, const float* D_skip, const void* z,
                     const float* delta_bias, int flags, void* y, int batch, int dim,
                     int dstate, int dtype, void* stream) {
  return update_impl(state, u, delta, A, B, C, D_skip, z, delta_bias, flags, y, batch, dim, dstate,
                     dtype, stream, nullptr);
}

int ssm_conv_state_update(float* conv_state, float* state, const void* x, const float* conv_w,
                          const float* conv_b, int conv_width, const void* delta, const float* A,
                          const void* B, const void* C, const float* D_skip, const void* z,
                          const float* delta_bias, int flags, void* y, int batch, int dim,
                          int dstate, int dtype, void* stream) {
  const ConvIn cv{conv_w, conv_b, nullptr, nullptr, conv_state, conv_width};
  return update_impl(state, x, delta, A, B, C, D_skip, z, delta_bias, flags, y, batch, dim, dstate,
                     dtype, stream, &cv);
}

size_t ssm_scan_bwd_workspace_bytes(int batch, int dim, int dstate, int64_t seqlen, int dtype) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return 0;
  if (!dstate_ok(dstate) || !shapes_fit(batch, dim, seqlen)) return 0;
  if (batch == 0 || dim == 0 || seqlen == 0) return 0;
  return bwd_workspace_layout(batch, dim, dstate, seqlen, dtype,
                              plan_segments(batch, dim, dstate, seqlen, dtype))
      .total;
}

// ckpt_given: the checkpoints come from the caller (ckpt_in, written by
// ssm_scan_fwd_ckpt), so the forward checkpoint pass is skipped and only the
// B, C records are packed.
static int bwd_impl(const void* u, const void* delta, const float* A, const void* B, const void* C,
                    const float* D_skip, const void* z, const float* delta_bias, int flags,
                    const float* h0, const void* dy, const float* dlast_state, void* du, void* ddelta,
                    float* dA, void* dB, void* dC, float* dD, void* dz, float* ddelta_bias,
                    float* dh0, int batch, int dim, int dstate, int64_t seqlen, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream, bool ckpt_given,
                    const float* ckpt_in, size_t ckpt_bytes) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (!flags_ok(flags)) return SSM_ERR_FLAGS;
  if (!dstate_ok(dstate) || !shapes_fit(batch, dim, seqlen)) return SSM_ERR_SHAPE;
  const bool empty = batch == 0 || dim == 0;
  if (!empty && (!A || !dA)) return SSM_ERR_NULL;
  if (!empty && seqlen > 0 &&
      (!u || !delta || !B || !C || !dy || !du || !ddelta || !dB || !dC || (z != nullptr && !dz)))
    return SSM_ERR_NULL;
  const size_t es = (size_t)elem_bytes(dtype);
  if (!aligned(u, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) ||
      !aligned(z, es) || !aligned(dy, es) || !aligned(du, es) || !aligned(ddelta, es) ||
      !aligned(dB, es) || !aligned(dC, es) || !aligned(dz, es) || !aligned(A, 4) ||
      !aligned(D_skip, 4) || !aligned(delta_bias, 4) || !aligned(h0, 4) || !aligned(dlast_state, 4) ||
      !aligned(dA, 4) || !aligned(dD, 4) || !aligned(ddelta_bias, 4) || !aligned(dh0, 4) ||
      !aligned(workspace, 256) || !aligned(ckpt_in, 4))
    return SSM_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (empty) return SSM_OK;
  const size_t ckb = ckpt_given ? ckpt_bytes_of(batch, dim, dstate, seqlen) : 0;
  if (ckb > 0 && ckpt_in == nullptr) return SSM_ERR_NULL;
  if (ckb > 0 && ckpt_bytes < ckb) return SSM_ERR_WORKSPACE;
  {
    const size_t tok = (size_t)batch * (size_t)dim * (size_t)seqlen * es;
    const size_t bc = (size_t)batch * (size_t)dstate * (size_t)seqlen * es;
    const size_t per_dim = (size_t)dim * sizeof(float);
    const size_t state = (size_t)batch * (size_t)dim * (size_t)dstate * sizeof(float);
    const Span outs[] = {span(du, tok), span(ddelta, tok), span(dz, tok), span(dB, bc), span(dC, bc),
                         span(dA, per_dim * (size_t)dstate), span(dD, per_dim),
                         span(ddelta_bias, per_dim), span(dh0, state)};
    const Span ins[] = {span(u, tok), span(delta, tok), span(z, tok), span(dy, tok), span(B, bc),
                        span(C, bc), span(A, per_dim * (size_t)dstate), span(D_skip, per_dim),
                        span(delta_bias, per_dim), span(h0, state), span(dlast_state, state),
                        span(ckpt_in, ckb)};
    if (writes_overlap(outs, ins)) return SSM_ERR_ALIAS;
  }

  if (seqlen == 0) {  // no steps: zero parameter gradients, dh0 = dlast
    hipError_t e = ssm::launch_fill_state(dA, nullptr, (int64_t)dim * dstate, st);
    if (e == hipSuccess && dD != nullptr) e = ssm::launch_fill_state(dD, nullptr, dim, st);
    if (e == hipSuccess && ddelta_bias != nullptr)
      e = ssm::launch_fill_state(ddelta_bias, nullptr, dim, st);
    if (e == hipSuccess && dh0 != nullptr)
      e = ssm::launch_fill_state(dh0, dlast_state, (int64_t)batch * dim * dstate, st);
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
  }

  const SegPlan sp = plan_segments(batch, dim, dstate, seqlen, dtype);
  const int64_t blocks = (int64_t)batch * ((dim + 63) / 64) * sp.nseg;
  const int64_t pack_blocks = (int64_t)batch * ((seqlen + 255) / 256);
  const int64_t red_blocks = (2 * (int64_t)batch * dstate * seqlen + 255) / 256;
  if (blocks > INT_MAX || pack_blocks > INT_MAX || red_blocks > INT_MAX) return SSM_ERR_SHAPE;
  const BwdWsLayout wl = bwd_workspace_layout(batch, dim, dstate, seqlen, dtype, sp, !ckpt_given);
  if (workspace == nullptr || workspace_bytes < wl.total) return SSM_ERR_WORKSPACE;
  {
    const size_t tok = (size_t)batch * (size_t)dim * (size_t)seqlen * es;
    const size_t bc = (size_t)batch * (size_t)dstate * (size_t)seqlen * es;
    const size_t per_dim = (size_t)dim * sizeof(float);
    const size_t state = (size_t)batch * (size_t)dim * (size_t)dstate * sizeof(float);
    const Span outs[] = {span(workspace, wl.total)};
    const Span ins[] = {span(u, tok), span(delta, tok), span(z, tok), span(dy, tok), span(B, bc),
                        span(C, bc), span(A, per_dim * (size_t)dstate), span(D_skip, per_dim),
                        span(delta_bias, per_dim), span(h0, state), span(dlast_state, state),
                        span(du, tok), span(ddelta, tok), span(dz, tok), span(dB, bc), span(dC, bc),
                        span(dA, per_dim * (size_t)dstate), span(dD, per_dim),
                        span(ddelta_bias, per_dim), span(dh0, state), span(ckpt_in, ckb)};
    if (writes_overlap(outs, ins)) return SSM_ERR_ALIAS;
  }
  char* ws = static_cast<char*>(workspace);
  const bool rows16 = ((int64_t)es * seqlen) % 16 == 0;

  // 1. forward checkpoint pass (packs the B, C records too)
  ssm::ScanLaunch f{};
  f.u = u;
  f.delta = delta;
  f.A = A;
  f.B = B;
  f.C = C;
  f.Dskip = D_skip;
  f.bias = delta_bias;
  f.h0 = h0;
  f.ws_bc = ws + wl.fwd.bc;
  if (sp.nseg > 1) {
    f.ws_hend = reinterpret_cast<float*>(ws + wl.fwd.hend);
    f.ws_sumdt = reinterpret_cast<float*>(ws + wl.fwd.sumdt);
  }
  f.batch = batch;
  f.dim = dim;
  f.dstate = dstate;
  f.seqlen = seqlen;
  f.seglen = sp.seglen;
  f.nseg = sp.nseg;
  f.softplus = (flags & SSM_DELTA_SOFTPLUS) ? 1 : 0;
  f.zoh = (flags & SSM_BBAR_ZOH) ? 1 : 0;
  f.vec = rows16 && group_rows_fit(seqlen, es) && aligned(u, 16) && aligned(delta, 16);
  f.dtype = dtype == SSM_BF16 ? Dtype::BF16 : Dtype::F32;
  f.ncu = device_cu_count();
  f.prio_blocks = prio_blocks();
  if (ckpt_given) {
    if (ssm::launch_pack_records(f, st) != hipSuccess) return SSM_ERR_HIP;
  } else {
    f.ws_ckpt = reinterpret_cast<float*>(ws + wl.ckpt);
    if (ssm::launch_scan_fwd(f, st) != hipSuccess) return SSM_ERR_HIP;
  }

  // 2-4. reverse aggregates, the backward sweep, the sums of the partials
  ssm::BwdLaunch a{};
  a.u = u;
  a.delta = delta;
  a.A = A;
  a.Dskip = D_skip;
  a.z = z;
  a.bias = delta_bias;
  a.dy = dy;
  a.dlast = dlast_state;
  a.du = du;
  a.ddelta = ddelta;
  a.dz = dz;
  a.dh0 = dh0;
  a.dA = dA;
  a.dB = dB;
  a.dC = dC;
  a.dD = dD;
  a.dbias = ddelta_bias;
  a.ws_bc = ws + wl.fwd.bc;
  a.ws_ckpt = ckpt_given ? ckpt_in : reinterpret_cast<const float*>(ws + wl.ckpt);
  a.ws_lagg = reinterpret_cast<float*>(ws + wl.lagg);
  a.ws_lsum = reinterpret_cast<float*>(ws + wl.lsum);
  a.ws_part_bc = reinterpret_cast<float*>(ws + wl.part_bc);
  a.ws_part_a = reinterpret_cast<float*>(ws + wl.part_a);
  a.ws_part_d = reinterpret_cast<float*>(ws + wl.part_d);
  a.ws_part_bias = reinterpret_cast<float*>(ws + wl.part_bias);
  a.batch = batch;
  a.dim = dim;
  a.dstate = dstate;
  a.seqlen = seqlen;
  a.seglen = sp.seglen;
  a.nseg = sp.nseg;
  a.softplus = f.softplus;
  a.zoh = f.zoh;
  a.vec = rows16 && group_rows_fit(seqlen, es) && aligned(u, 16) && aligned(delta, 16) && aligned(z, 16) &&
          aligned(dy, 16) && aligned(du, 16) && aligned(ddelta, 16) && aligned(dz, 16);
  a.dtype = f.dtype;
  return ssm::launch_scan_bwd(a, st) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                 const float* D_skip, const void* z, const float* delta_bias, int flags,
                 const float* h0, const void* dy, const float* dlast_state, void* du, void* ddelta,
                 float* dA, void* dB, void* dC, float* dD, void* dz, float* ddelta_bias,
                 float* dh0, int batch, int dim, int dstate, int64_t seqlen, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(u, delta, A, B, C, D_skip, z, delta_bias, flags, h0, dy, dlast_state, du, ddelta,
                  dA, dB, dC, dD, dz, ddelta_bias, dh0, batch, dim, dstate, seqlen, dtype, workspace,
                  workspace_bytes, stream, false, nullptr, 0);
}

size_t ssm_scan_ckpt_bytes(int batch, int dim, int dstate, int64_t seqlen) {
  if (!dstate_ok(dstate) || !shapes_fit(batch, dim, seqlen)) return 0;
  return ckpt_bytes_of(batch, dim, dstate, seqlen);
}

int ssm_scan_fwd_ckpt(const void* u, const void* delta, const float* A, const void* B, const void* C,
                      const float* D_skip, const void* z, const float* delta_bias, int flags,
                      const float* h0, void* y, float* last_state, float* ckpt, size_t ckpt_bytes,
                      int batch, int dim, int dstate, int64_t seqlen, int dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return scan_impl(u, delta, A, B, C, D_skip, z, delta_bias, flags, h0, y, last_state, batch, dim,
                   dstate, seqlen, dtype, workspace, workspace_bytes, stream, nullptr, false, true, ckpt,
                   ckpt_bytes);
}

size_t ssm_scan_bwd_ckpt_workspace_bytes(int batch, int dim, int dstate, int64_t seqlen, int dtype) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return 0;
  if (!dstate_ok(dstate) || !shapes_fit(batch, dim, seqlen)) return 0;
  if (batch == 0 || dim == 0 || seqlen == 0) return 0;
  return bwd_workspace_layout(batch, dim, dstate, seqlen, dtype,
                              plan_segments(batch, dim, dstate, seqlen, dtype), false)
      .total;
}

int ssm_scan_bwd_ckpt(const void* u, const void* delta, const float* A, const void* B, const void* C,
                      const float* D_skip, const void* z, const float* delta_bias, int flags,
                      const float* h0, const float* ckpt, size_t ckpt_bytes, const void* dy,
                      const float* dlast_state, void* du, void* ddelta, float* dA, void* dB, void* dC,
                      float* dD, void* dz, float* ddelta_bias, float* dh0, int batch, int dim,
                      int dstate, int64_t seqlen, int dtype, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return bwd_impl(u, delta, A, B, C, D_skip, z, delta_bias, flags, h0, dy, dlast_state, du, ddelta,
                  dA, dB, dC, dD, dz, ddelta_bias, dh0, batch, dim, dstate, seqlen, dtype, workspace,
                  workspace_bytes, stream, true, ckpt, ckpt_bytes);
}

size_t ssm_ssd_scan_fwd_workspace_bytes(int batch, int dstate, int64_t seqlen, int dtype) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return 0;
  if (batch <= 0 || seqlen <= 0 || dstate <= 0 || dstate > 128) return 0;
  return ssm::ssd_ws_bytes(batch, dstate, seqlen, elem_bytes(dtype));
}

int ssm_ssd_scan_fwd(const void* x, const void* dt, const float* A_head, const void* B,
                     const void* C, const float* D_skip, const void* z, const float* dt_bias,
                     int flags, const float* h0, void* y, float* last_state, int batch, int nheads,
                     int headdim, int dstate, int64_t seqlen, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (!flags_ok(flags)) return SSM_ERR_FLAGS;
  if (batch < 0 || nheads < 0 || seqlen < 0) return SSM_ERR_SHAPE;
  if (headdim != ssm::kSsdHeadDim) return SSM_ERR_SHAPE;
  const bool n_ok = dstate == 16 || dstate == 32 || dstate == 64 || (dstate == 128 && dtype == SSM_BF16);
  if (!n_ok) return SSM_ERR_SHAPE;
  if ((int64_t)nheads * headdim > INT_MAX / 2 || !shapes_fit(batch, nheads * headdim, seqlen))
    return SSM_ERR_SHAPE;
  if ((int64_t)batch * nheads > INT_MAX) return SSM_ERR_SHAPE;
  const bool empty = batch == 0 || nheads == 0;
  if (!empty && seqlen > 0 && (!x || !dt || !A_head || !B || !C || !y)) return SSM_ERR_NULL;
  const size_t es = (size_t)elem_bytes(dtype);
  if (!aligned(x, es) || !aligned(dt, es) || !aligned(B, es) || !aligned(C, es) ||
      !aligned(z, es) || !aligned(y, es) || !aligned(A_head, 4) || !aligned(D_skip, 4) ||
      !aligned(dt_bias, 4) || !aligned(h0, 4) || !aligned(last_state, 4) || !aligned(workspace, 256))
    return SSM_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (empty) return SSM_OK;
  if (seqlen == 0) {
    if (last_state == nullptr) return SSM_OK;
    const hipError_t e =
        ssm::launch_fill_state(last_state, h0, (int64_t)batch * nheads * headdim * dstate, st);
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
  }
  if ((int64_t)batch * ((seqlen + 63) / 64) > INT_MAX) return SSM_ERR_SHAPE;
  // the kernel addresses a head's x, z, y rows, a batch row's B, C^T and its
  // chunk tiles with 32-bit byte offsets
  const int64_t widest = dstate > ssm::kSsdHeadDim ? dstate : ssm::kSsdHeadDim;
  if (seqlen * widest * (int64_t)es > INT_MAX || (seqlen + 63) / 64 * 10240 > INT_MAX) return SSM_ERR_SHAPE;
  const size_t ssd_tok = (size_t)batch * (size_t)nheads * (size_t)headdim * (size_t)seqlen * es;
  const size_t ssd_bc = (size_t)batch * (size_t)dstate * (size_t)seqlen * es;
  const size_t ssd_state = (size_t)batch * (size_t)nheads * (size_t)headdim * (size_t)dstate * 4;
  {
    const Span outs[] = {span(y, ssd_tok), span(last_state, ssd_state)};
    const Span ins[] = {span(x, ssd_tok), span(z, ssd_tok),
                        span(dt, (size_t)batch * (size_t)nheads * (size_t)seqlen * es),
                        span(B, ssd_bc), span(C, ssd_bc), span(A_head, (size_t)nheads * 4),
                        span(D_skip, (size_t)nheads * (size_t)headdim * 4),
                        span(dt_bias, (size_t)nheads * 4), span(h0, ssd_state)};
    if (writes_overlap(outs, ins)) return SSM_ERR_ALIAS;
  }
  const size_t ssd_ws = ssm_ssd_scan_fwd_workspace_bytes(batch, dstate, seqlen, dtype);
  if (workspace == nullptr || workspace_bytes < ssd_ws) return SSM_ERR_WORKSPACE;
  {
    const Span outs[] = {span(workspace, ssd_ws)};
    const Span ins[] = {span(x, ssd_tok), span(z, ssd_tok),
                        span(dt, (size_t)batch * (size_t)nheads * (size_t)seqlen * es),
                        span(B, ssd_bc), span(C, ssd_bc), span(A_head, (size_t)nheads * 4),
                        span(D_skip, (size_t)nheads * (size_t)headdim * 4),
                        span(dt_bias, (size_t)nheads * 4), span(h0, ssd_state), span(y, ssd_tok),
                        span(last_state, ssd_state)};
    if (writes_overlap(outs, ins)) return SSM_ERR_ALIAS;
  }
  ssm::SsdLaunch a{};
  a.x = x;
  a.dt = dt;
  a.A = A_head;
  a.B = B;
  a.C = C;
  a.Dskip = D_skip;
  a.z = z;
  a.dt_bias = dt_bias;
  a.h0 = h0;
  a.y = y;
  a.last_state = last_state;
  a.ws = workspace;
  a.batch = batch;
  a.nheads = nheads;
  a.headdim = headdim;
  a.dstate = dstate;
  a.seqlen = seqlen;
  a.softplus = (flags & SSM_DELTA_SOFTPLUS) ? 1 : 0;
  a.zoh = (flags & SSM_BBAR_ZOH) ? 1 : 0;
  const bool rows16 = ((int64_t)es * seqlen) % 16 == 0;
  a.vec = rows16 && aligned(x, 16) && aligned(B, 16) && aligned(C, 16) && aligned(z, 16) &&
          aligned(y, 16);
  a.dtype = dtype == SSM_BF16 ? Dtype::BF16 : Dtype::F32;
  return ssm::launch_ssd_fwd(a, st) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

const char* ssm_status_string(int status) {
  switch (status) {
    case SSM_OK: return "SSM_OK";
    case SSM_ERR_NULL: return "SSM_ERR_NULL: a required pointer is NULL";
    case SSM_ERR_SHAPE: return "SSM_ERR_SHAPE: bad or too large sizes, or dstate not in {1,2,4,8,16}";
    case SSM_ERR_DTYPE: return "SSM_ERR_DTYPE: dtype is not SSM_F32 or SSM_BF16";
    case SSM_ERR_ALIGN: return "SSM_ERR_ALIGN: a pointer is not aligned to its element size";
    case SSM_ERR_WORKSPACE: return "SSM_ERR_WORKSPACE: workspace missing or too small";
    case SSM_ERR_HIP: return "SSM_ERR_HIP: the HIP runtime reported a launch error";
    case SSM_ERR_ALIAS: return "SSM_ERR_ALIAS: a buffer the call writes overlaps another buffer of the call";
    case SSM_ERR_FLAGS: return "SSM_ERR_FLAGS: flags holds an unknown bit";
    case kStatusScratch:
      return "SSM_ERR_SCRATCH: the problem needs more workspace than the 16 MiB static scratch of "
             "ssm_scan_fwd_noalloc holds (ssm_scan_fwd_workspace_bytes gives the need)";
    default: return "unknown ssm status";
  }
}

}  // extern "C"
