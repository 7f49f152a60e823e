// ssm_api.cpp -- the C ABI of libssm (declared in include/ssm.h): argument
// validation, choice of the launch plan, and the calls into the kernels.
//
// Every check happens before the first HIP call, so a rejected call enqueues
// nothing and the validation can be exercised without a GPU.
#include <climits>
#include <cstdint>
#include <cstdlib>

#include "ssm.h"
#include "ssm_kernels.hpp"

namespace {

using ssm::Dtype;

// A launch should put about four waves on each of the 1024 SIMDs of a
// 256-CU gfx950 before the sequence is split into segments; a segment is never
// shorter than kMinSegment steps unless a caller forces the split.
constexpr int64_t kTargetWaves = 4096;
constexpr int64_t kMinSegment = 512;

struct SegPlan {
  int nseg;
  int64_t seglen;
};

bool dstate_ok(int n) { return n == 1 || n == 2 || n == 4 || n == 8 || n == 16; }

int elem_bytes(int dtype) { return dtype == SSM_BF16 ? 2 : 4; }

// Segments of the sequence for the forward scan.  SSM_SCAN_SEGMENTS (an
// integer >= 1) overrides the choice; tests use it to run the carry path at
// small sizes.
SegPlan plan_segments(int batch, int dim, int dstate, int64_t L) {
  const int64_t tile = ssm::kScanTile;
  const int64_t G = dstate >= 4 ? dstate / 4 : 1;
  const int64_t ncg = (dim + 63) / 64;
  const int64_t waves = (int64_t)batch * ncg * G;
  int64_t want = waves > 0 ? (kTargetWaves + waves - 1) / waves : 1;
  int64_t cap = L / kMinSegment;
  if (const char* env = std::getenv("SSM_SCAN_SEGMENTS")) {
    const long long v = std::atoll(env);
    if (v >= 1) {
      want = v;
      cap = want;
    }
  }
  if (want > cap) want = cap;
  const int64_t tiles = (L + tile - 1) / tile;
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  int64_t seglen = (L + want - 1) / want;
  seglen = (seglen + tile - 1) / tile * tile;
  if (seglen < tile) seglen = tile;
  const int64_t nseg = (L + seglen - 1) / seglen;
  return SegPlan{(int)(nseg < 1 ? 1 : nseg), seglen};
}

size_t workspace_for(int batch, int dim, int dstate, const SegPlan& sp) {
  if (sp.nseg <= 1) return 0;
  const size_t plane = (size_t)batch * (size_t)dim;
  const size_t hend = (size_t)(sp.nseg - 1) * plane * (size_t)dstate * sizeof(float);
  const size_t sumdt = (size_t)(sp.nseg - 1) * plane * sizeof(float);
  return ((hend + 255) / 256) * 256 + sumdt;
}

bool aligned(const void* p, size_t a) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool shapes_fit(int batch, int dim, int64_t seqlen) {
  if (batch < 0 || dim < 0 || seqlen < 0) return false;
  const long double total = (long double)batch * (long double)dim * (long double)(seqlen > 0 ? seqlen : 1);
  return total < (long double)(INT64_C(1) << 60);
}

}  // namespace

extern "C" {

size_t ssm_scan_fwd_workspace_bytes(int batch, int dim, int dstate, int64_t seqlen, int dtype) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return 0;
  if (!dstate_ok(dstate) || !shapes_fit(batch, dim, seqlen)) return 0;
  if (batch == 0 || dim == 0 || seqlen == 0) return 0;
  return workspace_for(batch, dim, dstate, plan_segments(batch, dim, dstate, seqlen));
}

int ssm_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                 const float* D_skip, const void* z, const float* delta_bias, int delta_softplus,
                 const float* h0, void* y, float* last_state, int batch, int dim, int dstate,
                 int64_t seqlen, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (!dstate_ok(dstate) || !shapes_fit(batch, dim, seqlen)) return SSM_ERR_SHAPE;
  const bool empty = batch == 0 || dim == 0;
  if (!empty && seqlen > 0 && (!u || !delta || !A || !B || !C || !y)) return SSM_ERR_NULL;
  const size_t es = (size_t)elem_bytes(dtype);
  if (!aligned(u, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) ||
      !aligned(z, es) || !aligned(y, es) || !aligned(A, 4) || !aligned(D_skip, 4) ||
      !aligned(delta_bias, 4) || !aligned(h0, 4) || !aligned(last_state, 4) ||
      !aligned(workspace, 4))
    return SSM_ERR_ALIGN;
  if (y != nullptr && (y == u || y == delta || (z != nullptr && y == z))) return SSM_ERR_ALIAS;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (empty) return SSM_OK;

  if (seqlen == 0) {  // nothing to scan: the state stays h0 (or zero)
    if (last_state == nullptr) return SSM_OK;
    const hipError_t e = ssm::launch_fill_state(last_state, h0, (int64_t)batch * dim * dstate, st);
    return e == hipSuccess ? SSM_OK : SSM_ERR_HIP;
  }

  const SegPlan sp = plan_segments(batch, dim, dstate, seqlen);
  const int64_t blocks = (int64_t)batch * ((dim + 63) / 64) * sp.nseg;
  if (blocks > INT_MAX) return SSM_ERR_SHAPE;
  const size_t need = workspace_for(batch, dim, dstate, sp);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return SSM_ERR_WORKSPACE;

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
  if (need > 0) {
    const size_t plane = (size_t)batch * (size_t)dim;
    const size_t hend = (size_t)(sp.nseg - 1) * plane * (size_t)dstate * sizeof(float);
    a.ws_hend = static_cast<float*>(workspace);
    a.ws_sumdt = reinterpret_cast<float*>(static_cast<char*>(workspace) + ((hend + 255) / 256) * 256);
  }
  a.batch = batch;
  a.dim = dim;
  a.dstate = dstate;
  a.seqlen = seqlen;
  a.seglen = sp.seglen;
  a.nseg = sp.nseg;
  a.softplus = delta_softplus ? 1 : 0;
  const bool rows16 = ((int64_t)es * seqlen) % 16 == 0;
  a.vec = rows16 && aligned(u, 16) && aligned(delta, 16) && aligned(z, 16) && aligned(y, 16);
  a.dtype = dtype == SSM_BF16 ? Dtype::BF16 : Dtype::F32;
  return ssm::launch_scan_fwd(a, st) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

int ssm_state_update(float* state, const void* u, const void* delta, const float* A,
                     const void* B, const void* C, const float* D_skip, const void* z,
                     const float* delta_bias, int delta_softplus, void* y, int batch, int dim,
                     int dstate, int dtype, void* stream) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (!dstate_ok(dstate) || !shapes_fit(batch, dim, 1)) return SSM_ERR_SHAPE;
  const bool empty = batch == 0 || dim == 0;
  if (!empty && (!state || !u || !delta || !A || !B || !C || !y)) return SSM_ERR_NULL;
  const size_t es = (size_t)elem_bytes(dtype);
  if (!aligned(state, 4) || !aligned(u, es) || !aligned(delta, es) || !aligned(B, es) ||
      !aligned(C, es) || !aligned(z, es) || !aligned(y, es) || !aligned(A, 4) ||
      !aligned(D_skip, 4) || !aligned(delta_bias, 4))
    return SSM_ERR_ALIGN;
  if (y != nullptr && (y == u || y == delta || y == state || (z != nullptr && y == z)))
    return SSM_ERR_ALIAS;
  if (empty) return SSM_OK;
  const int64_t threads = (int64_t)batch * dim * (dstate >= 4 ? dstate / 4 : 1);
  if ((threads + 255) / 256 > INT_MAX) return SSM_ERR_SHAPE;

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
  a.softplus = delta_softplus ? 1 : 0;
  a.vec = aligned(state, 16) ? 1 : 0;
  a.dtype = dtype == SSM_BF16 ? Dtype::BF16 : Dtype::F32;
  return ssm::launch_state_update(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SSM_OK
                                                                                    : SSM_ERR_HIP;
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
    case SSM_ERR_ALIAS: return "SSM_ERR_ALIAS: an output is the same buffer as an input";
    default: return "unknown ssm status";
  }
}

}  // extern "C"
