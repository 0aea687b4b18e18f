// C-ABI entry points of libmambascan: host-side validation, then launch.
// Everything here runs on the host before any HIP call; on any error nothing
// is enqueued and no output is touched.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/mambascan.h"
#include "launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(mss_dtype t) { return t == MSS_BF16 ? 2 : 4; }

bool dtype_ok(mss_dtype t) { return t == MSS_FP32 || t == MSS_BF16; }

// An output range must not overlap any of the listed (non-null) input ranges.
bool output_clear(const void* out, size_t out_bytes, const void* const* ins, const size_t* in_bytes, int n) {
  if (out == nullptr) return true;
  const Range o = range_of(out, out_bytes);
  for (int i = 0; i < n; ++i)
    if (ins[i] != nullptr && overlaps(o, range_of(ins[i], in_bytes[i]))) return false;
  return true;
}

mss_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MSS_OK;
  g_last_hip_error = static_cast<int>(e);
  return MSS_ERR_HIP;
}

constexpr int64_t kMaxIndex = INT32_MAX;

// Scratch of mss_selective_scan_fwd_noalloc, for callers that cannot allocate:
// one copy per GPU, held until the process ends.  In host code `scratch`
// names a host-side stand-in; its device address, different on each GPU,
// comes from hipGetSymbolAddress with that GPU current and is kept per device.
constexpr size_t kNoAllocScratchBytes = size_t{64} << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, looked up on its first use there.
hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* mss_status_string(mss_status s) {
  switch (s) {
    case MSS_OK: return "MSS_OK";
    case MSS_ERR_NULL: return "MSS_ERR_NULL: a required pointer is NULL";
    case MSS_ERR_SHAPE: return "MSS_ERR_SHAPE: a size is not positive or is too large";
    case MSS_ERR_DTYPE: return "MSS_ERR_DTYPE: unknown dtype";
    case MSS_ERR_ALIGN: return "MSS_ERR_ALIGN: a pointer is not 16-byte aligned";
    case MSS_ERR_UNSUPPORTED: return "MSS_ERR_UNSUPPORTED: shape or option not implemented";
    case MSS_ERR_WORKSPACE: return "MSS_ERR_WORKSPACE: workspace missing or too small";
    case MSS_ERR_ALIAS: return "MSS_ERR_ALIAS: an output overlaps an input";
    case MSS_ERR_HIP: return "MSS_ERR_HIP: a HIP call failed";
    case MSS_ERR_WAIT: return "MSS_ERR_WAIT: a bounded wait between workgroups gave up; the outputs are not valid";
  }
  return "unknown mss_status";
}

int mss_last_hip_error(void) { return g_last_hip_error; }

int mss_abi_version(void) { return MSS_ABI_VERSION; }

mss_status mss_workspace_status(const void* workspace, void* hip_stream) {
  if (workspace == nullptr) return MSS_ERR_NULL;
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(hip_stream));
  int word = 0;
  if (e == hipSuccess) e = hipMemcpy(&word, workspace, sizeof(word), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_status(e);
  return word == 0 ? MSS_OK : MSS_ERR_WAIT;
}

// ------------------------------------------------------------ selective scan
static mss_status scan_check_shape(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, mss_dtype t) {
  if (!dtype_ok(t)) return MSS_ERR_DTYPE;
  if (batch <= 0 || dim <= 0 || dstate <= 0 || seqlen <= 0) return MSS_ERR_SHAPE;
  if (batch > 65535 || seqlen >= (1LL << 24) || dim * seqlen > kMaxIndex || dim * dstate > kMaxIndex ||
      batch * dim > kMaxIndex)
    return MSS_ERR_SHAPE;
  if (dstate > 128) return MSS_ERR_UNSUPPORTED;
  return MSS_OK;
}

size_t mss_selective_scan_workspace_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                         mss_dtype io_dtype, uint32_t flags) {
  (void)flags;
  if (scan_check_shape(batch, dim, dstate, seqlen, io_dtype) != MSS_OK) return 0;
  return mss::scan_workspace_bytes(batch, dim, dstate, seqlen);
}

// The selective scan forward's checks before the workspace's: pointers,
// shape, flags, alignment (`extra`, a 4-byte output, only needs 4 bytes).
static mss_status scan_fwd_check_args(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                      const float* D, const void* z, const float* h0, const void* y,
                                      const float* h_last, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                      mss_dtype io_dtype, uint32_t flags, const void* workspace, const void* extra) {
  if (!u || !delta || !A || !B || !C || !y) return MSS_ERR_NULL;
  mss_status st = scan_check_shape(batch, dim, dstate, seqlen, io_dtype);
  if (st != MSS_OK) return st;
  if (flags & ~MSS_FLAG_DECAY_GENERAL) return MSS_ERR_UNSUPPORTED;
  const void* all[] = {u, delta, A, B, C, D, z, h0, y, h_last, workspace};
  for (const void* p : all)
    if (p && !aligned16(p)) return MSS_ERR_ALIGN;
  if (extra && (reinterpret_cast<uintptr_t>(extra) & 3u)) return MSS_ERR_ALIGN;
  return MSS_OK;
}

// ... and after it: no output overlaps an input (the workspace, `need` bytes,
// counts as one) or another output (`extra`, 4 bytes, nullable).
static mss_status scan_fwd_check_alias(const void* u, const void* delta, const float* A, const void* B,
                                       const void* C, const float* D, const void* z, const float* h0, const void* y,
                                       const float* h_last, int64_t batch, int64_t dim, int64_t dstate,
                                       int64_t seqlen, mss_dtype io_dtype, const void* workspace, size_t need,
                                       const void* extra) {
  const size_t es = elem_size(io_dtype);
  const size_t nbdl = (size_t)batch * dim * seqlen;
  const size_t nbnl = (size_t)batch * dstate * seqlen;
  const size_t nstate = (size_t)batch * dim * dstate * sizeof(float);
  const void* ins[] = {u, delta, A, B, C, D, z, h0, workspace};
  const size_t in_bytes[] = {nbdl * es, nbdl * es, (size_t)dim * dstate * 4, nbnl * es, nbnl * es,
                             (size_t)dim * 4, nbdl * es, nstate, need};
  if (!output_clear(y, nbdl * es, ins, in_bytes, 9)) return MSS_ERR_ALIAS;
  if (!output_clear(h_last, nstate, ins, in_bytes, 9)) return MSS_ERR_ALIAS;
  if (h_last && overlaps(range_of(y, nbdl * es), range_of(h_last, nstate))) return MSS_ERR_ALIAS;
  if (extra) {
    const Range e = range_of(extra, sizeof(int));
    if (!output_clear(extra, sizeof(int), ins, in_bytes, 9)) return MSS_ERR_ALIAS;
    if (overlaps(e, range_of(y, nbdl * es))) return MSS_ERR_ALIAS;
    if (h_last && overlaps(e, range_of(h_last, nstate))) return MSS_ERR_ALIAS;
  }
  return MSS_OK;
}

static mss::ScanParams scan_params(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                   const float* D, const void* z, const float* h0, void* y, float* h_last,
                                   int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, mss_dtype io_dtype,
                                   uint32_t flags, void* workspace) {
  mss::ScanParams p;
  p.u = u;
  p.delta = delta;
  p.A = A;
  p.B = B;
  p.C = C;
  p.D = D;
  p.z = z;
  p.h0 = h0;
  p.y = y;
  p.h_last = h_last;
  p.batch = batch;
  p.dim = dim;
  p.dstate = dstate;
  p.seqlen = seqlen;
  p.bf16 = io_dtype == MSS_BF16;
  p.force_general = (flags & MSS_FLAG_DECAY_GENERAL) != 0;
  p.workspace = workspace;
  return p;
}

mss_status mss_selective_scan_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                  const float* D, const void* z, const float* h0, void* y, float* h_last,
                                  int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, mss_dtype io_dtype,
                                  uint32_t flags, void* workspace, size_t workspace_bytes, void* hip_stream) {
  mss_status st = scan_fwd_check_args(u, delta, A, B, C, D, z, h0, y, h_last, batch, dim, dstate, seqlen, io_dtype,
                                      flags, workspace, nullptr);
  if (st != MSS_OK) return st;
  const size_t need = mss::scan_workspace_bytes(batch, dim, dstate, seqlen);
  if (!workspace || workspace_bytes < need) return MSS_ERR_WORKSPACE;
  st = scan_fwd_check_alias(u, delta, A, B, C, D, z, h0, y, h_last, batch, dim, dstate, seqlen, io_dtype, workspace,
                            need, nullptr);
  if (st != MSS_OK) return st;
  const mss::ScanParams p = scan_params(u, delta, A, B, C, D, z, h0, y, h_last, batch, dim, dstate, seqlen, io_dtype,
                                        flags, workspace);
  return hip_status(mss::launch_scan(p, static_cast<hipStream_t>(hip_stream)));
}

mss_status mss_selective_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B,
                                          const void* C, const float* D, const void* z, const float* h0, void* y,
                                          float* h_last, int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                          mss_dtype io_dtype, uint32_t flags, int* wait_status, void* hip_stream) {
  mss_status st = scan_fwd_check_args(u, delta, A, B, C, D, z, h0, y, h_last, batch, dim, dstate, seqlen, io_dtype,
                                      flags, nullptr, wait_status);
  if (st != MSS_OK) return st;
  st = scan_fwd_check_alias(u, delta, A, B, C, D, z, h0, y, h_last, batch, dim, dstate, seqlen, io_dtype, nullptr, 0,
                            wait_status);
  if (st != MSS_OK) return st;
  if (mss::scan_workspace_bytes(batch, dim, dstate, seqlen) > kNoAllocScratchBytes) return MSS_ERR_WORKSPACE;
  void* ws = nullptr;
  const hipError_t e = scratch_of_current_device(&ws);
  if (e != hipSuccess) return hip_status(e);
  mss::ScanParams p = scan_params(u, delta, A, B, C, D, z, h0, y, h_last, batch, dim, dstate, seqlen, io_dtype, flags,
                                  ws);
  p.status = wait_status;
  return hip_status(mss::launch_scan(p, static_cast<hipStream_t>(hip_stream)));
}

mss_status mss_selective_scan_fwd_fused(const void* x, const float* conv_w, const float* conv_b,
                                        const void* delta_raw, const float* delta_bias, const float* A,
                                        const void* B, const void* C, const float* D, const void* z,
                                        const float* h0, void* y, float* h_last, int64_t batch, int64_t dim,
                                        int64_t dstate, int64_t seqlen, mss_dtype io_dtype, uint32_t flags,
                                        void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!x || !conv_w || !delta_raw || !A || !B || !C || !y) return MSS_ERR_NULL;
  mss_status st = scan_check_shape(batch, dim, dstate, seqlen, io_dtype);
  if (st != MSS_OK) return st;
  if (flags & ~(MSS_FLAG_DECAY_GENERAL | MSS_FLAG_CONV_SILU | MSS_FLAG_DELTA_SOFTPLUS)) return MSS_ERR_UNSUPPORTED;
  const void* all[] = {x, conv_w, conv_b, delta_raw, delta_bias, A, B, C, D, z, h0, y, h_last, workspace};
  for (const void* p : all)
    if (p && !aligned16(p)) return MSS_ERR_ALIGN;
  const size_t need = mss::scan_workspace_bytes(batch, dim, dstate, seqlen);
  if (!workspace || workspace_bytes < need) return MSS_ERR_WORKSPACE;

  const size_t es = elem_size(io_dtype);
  const size_t nbdl = (size_t)batch * dim * seqlen;
  const size_t nbnl = (size_t)batch * dstate * seqlen;
  const size_t nstate = (size_t)batch * dim * dstate * sizeof(float);
  const void* ins[] = {x, conv_w, conv_b, delta_raw, delta_bias, A, B, C, D, z, h0, workspace};
  const size_t in_bytes[] = {nbdl * es, (size_t)dim * 16, (size_t)dim * 4, nbdl * es, (size_t)dim * 4,
                             (size_t)dim * dstate * 4, nbnl * es, nbnl * es, (size_t)dim * 4, nbdl * es, nstate,
                             need};
  if (!output_clear(y, nbdl * es, ins, in_bytes, 12)) return MSS_ERR_ALIAS;
  if (!output_clear(h_last, nstate, ins, in_bytes, 12)) return MSS_ERR_ALIAS;
  if (h_last && overlaps(range_of(y, nbdl * es), range_of(h_last, nstate))) return MSS_ERR_ALIAS;

  mss::ScanParams p;
  p.u = x;
  p.delta = delta_raw;
  p.A = A;
  p.B = B;
  p.C = C;
  p.D = D;
  p.z = z;
  p.h0 = h0;
  p.y = y;
  p.h_last = h_last;
  p.batch = batch;
  p.dim = dim;
  p.dstate = dstate;
  p.seqlen = seqlen;
  p.bf16 = io_dtype == MSS_BF16;
  p.force_general = (flags & MSS_FLAG_DECAY_GENERAL) != 0;
  p.workspace = workspace;
  p.fused = true;
  p.conv_w = conv_w;
  p.conv_b = conv_b;
  p.delta_bias = delta_bias;
  p.conv_silu = (flags & MSS_FLAG_CONV_SILU) != 0;
  p.delta_softplus = (flags & MSS_FLAG_DELTA_SOFTPLUS) != 0;
  return hip_status(mss::launch_scan(p, static_cast<hipStream_t>(hip_stream)));
}

// --------------------------------------------------- selective scan backward
// The forward's limits (d_state <= 128).  Up to 32 states the gradient
// kernels take them all (up to 4 states per wave); above, slices of 32 run
// one after the other.
static mss_status scan_bwd_check_shape(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen, mss_dtype t) {
  return scan_check_shape(batch, dim, dstate, seqlen, t);
}

static size_t scan_bwd_need(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen) {
  return dstate > 32 ? mss::scan_bwd_wide_workspace_bytes(batch, dim, seqlen)
                     : mss::scan_bwd_workspace_bytes(batch, dim, dstate, seqlen);
}

size_t mss_selective_scan_bwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                             mss_dtype io_dtype, uint32_t flags) {
  (void)flags;
  if (scan_bwd_check_shape(batch, dim, dstate, seqlen, io_dtype) != MSS_OK) return 0;
  return scan_bwd_need(batch, dim, dstate, seqlen);
}

mss_status mss_selective_scan_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                                  const float* D, const void* z, const float* h0, const void* dy,
                                  const float* dh_last, void* du, void* ddelta, float* dA, void* dB, void* dC,
                                  float* dD, void* dz, float* dh0, int64_t batch, int64_t dim, int64_t dstate,
                                  int64_t seqlen, mss_dtype io_dtype, uint32_t flags, void* workspace,
                                  size_t workspace_bytes, void* hip_stream) {
  if (!u || !delta || !A || !B || !C || !dy || !du || !ddelta || !dA || !dB || !dC) return MSS_ERR_NULL;
  if ((z == nullptr) != (dz == nullptr)) return MSS_ERR_NULL;
  mss_status st = scan_bwd_check_shape(batch, dim, dstate, seqlen, io_dtype);
  if (st != MSS_OK) return st;
  if (flags & ~MSS_FLAG_DECAY_GENERAL) return MSS_ERR_UNSUPPORTED;
  const void* all[] = {u, delta, A, B, C, D, z, h0, dy, dh_last, du, ddelta, dA, dB, dC, dD, dz, dh0, workspace};
  for (const void* p : all)
    if (p && !aligned16(p)) return MSS_ERR_ALIGN;
  const size_t need = scan_bwd_need(batch, dim, dstate, seqlen);
  if (!workspace || workspace_bytes < need) return MSS_ERR_WORKSPACE;

  const size_t es = elem_size(io_dtype);
  const size_t nbdl = (size_t)batch * dim * seqlen * es;
  const size_t nbnl = (size_t)batch * dstate * seqlen * es;
  const size_t nA = (size_t)dim * dstate * 4, nD = (size_t)dim * 4;
  const size_t nstate = (size_t)batch * dim * dstate * sizeof(float);
  const void* ins[] = {u, delta, A, B, C, D, z, h0, dy, dh_last, workspace};
  const size_t in_bytes[] = {nbdl, nbdl, nA, nbnl, nbnl, nD, nbdl, nstate, nbdl, nstate, need};
  void* outs[] = {du, ddelta, dA, dB, dC, dD, dz, dh0};
  const size_t out_bytes[] = {nbdl, nbdl, nA, nbnl, nbnl, nD, nbdl, nstate};
  for (int i = 0; i < 8; ++i) {
    if (!output_clear(outs[i], out_bytes[i], ins, in_bytes, 11)) return MSS_ERR_ALIAS;
    for (int j = i + 1; j < 8; ++j)
      if (outs[i] && outs[j] && overlaps(range_of(outs[i], out_bytes[i]), range_of(outs[j], out_bytes[j])))
        return MSS_ERR_ALIAS;
  }

  mss::ScanBwdParams p;
  p.fwd.u = u;
  p.fwd.delta = delta;
  p.fwd.A = A;
  p.fwd.B = B;
  p.fwd.C = C;
  p.fwd.D = D;
  p.fwd.z = z;
  p.fwd.h0 = h0;
  p.fwd.y = nullptr;
  p.fwd.h_last = nullptr;
  p.fwd.batch = batch;
  p.fwd.dim = dim;
  p.fwd.dstate = dstate;
  p.fwd.seqlen = seqlen;
  p.fwd.bf16 = io_dtype == MSS_BF16;
  p.fwd.force_general = (flags & MSS_FLAG_DECAY_GENERAL) != 0;
  p.fwd.workspace = workspace;
  p.dy = dy;
  p.dh_last = dh_last;
  p.du = du;
  p.ddelta = ddelta;
  p.dA = dA;
  p.dB = dB;
  p.dC = dC;
  p.dD = dD;
  p.dz = dz;
  p.dh0 = dh0;
  if (dstate > 32) return hip_status(mss::launch_scan_bwd_wide(p, static_cast<hipStream_t>(hip_stream)));
  return hip_status(mss::launch_scan_bwd(p, static_cast<hipStream_t>(hip_stream)));
}

// ------------------------------------------ fused scan (prologue) backward
size_t mss_selective_scan_fused_bwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                                   mss_dtype io_dtype, uint32_t flags) {
  (void)flags;
  if (scan_bwd_check_shape(batch, dim, dstate, seqlen, io_dtype) != MSS_OK) return 0;
  return mss::scan_fused_bwd_workspace_bytes(batch, dim, dstate, seqlen);
}

mss_status mss_selective_scan_fused_bwd(const void* x, const float* conv_w, const float* conv_b,
                                        const void* delta_raw, const float* delta_bias, const float* A,
                                        const void* B, const void* C, const float* D, const void* z,
                                        const float* h0, const void* dy, const float* dh_last, void* dx,
                                        void* ddelta_raw, float* dconv_w, float* dconv_b, float* ddelta_bias,
                                        float* dA, void* dB, void* dC, float* dD, void* dz, float* dh0,
                                        int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                        mss_dtype io_dtype, uint32_t flags, void* workspace, size_t workspace_bytes,
                                        void* hip_stream) {
  if (!x || !conv_w || !delta_raw || !A || !B || !C || !dy || !dx || !ddelta_raw || !dconv_w || !dA || !dB || !dC)
    return MSS_ERR_NULL;
  if ((z == nullptr) != (dz == nullptr)) return MSS_ERR_NULL;
  mss_status st = scan_bwd_check_shape(batch, dim, dstate, seqlen, io_dtype);
  if (st != MSS_OK) return st;
  if (flags & ~(MSS_FLAG_DECAY_GENERAL | MSS_FLAG_CONV_SILU | MSS_FLAG_DELTA_SOFTPLUS)) return MSS_ERR_UNSUPPORTED;
  const void* all[] = {x, conv_w, conv_b, delta_raw, delta_bias, A, B, C, D, z, h0, dy, dh_last, dx, ddelta_raw,
                       dconv_w, dconv_b, ddelta_bias, dA, dB, dC, dD, dz, dh0, workspace};
  for (const void* p : all)
    if (p && !aligned16(p)) return MSS_ERR_ALIGN;
  const size_t need = mss::scan_fused_bwd_workspace_bytes(batch, dim, dstate, seqlen);
  if (!workspace || workspace_bytes < need) return MSS_ERR_WORKSPACE;

  const size_t es = elem_size(io_dtype);
  const size_t nbdl = (size_t)batch * dim * seqlen * es;
  const size_t nbnl = (size_t)batch * dstate * seqlen * es;
  const size_t nA = (size_t)dim * dstate * 4, nD = (size_t)dim * 4;
  const size_t nstate = (size_t)batch * dim * dstate * sizeof(float);
  const void* ins[] = {x, conv_w, conv_b, delta_raw, delta_bias, A, B, C, D, z, h0, dy, dh_last, workspace};
  const size_t in_bytes[] = {nbdl, nD * 4, nD, nbdl, nD, nA, nbnl, nbnl, nD, nbdl, nstate, nbdl, nstate, need};
  void* outs[] = {dx, ddelta_raw, dconv_w, dconv_b, ddelta_bias, dA, dB, dC, dD, dz, dh0};
  const size_t out_bytes[] = {nbdl, nbdl, nD * 4, nD, nD, nA, nbnl, nbnl, nD, nbdl, nstate};
  for (int i = 0; i < 11; ++i) {
    if (!output_clear(outs[i], out_bytes[i], ins, in_bytes, 14)) return MSS_ERR_ALIAS;
    for (int j = i + 1; j < 11; ++j)
      if (outs[i] && outs[j] && overlaps(range_of(outs[i], out_bytes[i]), range_of(outs[j], out_bytes[j])))
        return MSS_ERR_ALIAS;
  }

  mss::ScanFusedBwdParams p;
  p.x = x;
  p.delta_raw = delta_raw;
  p.conv_w = conv_w;
  p.conv_b = conv_b;
  p.delta_bias = delta_bias;
  p.conv_silu = (flags & MSS_FLAG_CONV_SILU) != 0;
  p.softplus = (flags & MSS_FLAG_DELTA_SOFTPLUS) != 0;
  p.A = A;
  p.B = B;
  p.C = C;
  p.D = D;
  p.z = z;
  p.h0 = h0;
  p.dy = dy;
  p.dh_last = dh_last;
  p.dx = dx;
  p.ddelta_raw = ddelta_raw;
  p.dconv_w = dconv_w;
  p.dconv_b = dconv_b;
  p.ddelta_bias = ddelta_bias;
  p.dA = dA;
  p.dB = dB;
  p.dC = dC;
  p.dD = dD;
  p.dz = dz;
  p.dh0 = dh0;
  p.batch = batch;
  p.dim = dim;
  p.dstate = dstate;
  p.seqlen = seqlen;
  p.bf16 = io_dtype == MSS_BF16;
  p.force_general = (flags & MSS_FLAG_DECAY_GENERAL) != 0;
  p.workspace = workspace;
  return hip_status(mss::launch_scan_fused_bwd(p, static_cast<hipStream_t>(hip_stream)));
}

// -------------------------------------------------------------- state update
mss_status mss_state_update(float* h, const void* u, const void* delta, const float* A, const void* B,
                            const void* C, const float* D, const void* z, void* y, int64_t batch, int64_t dim,
                            int64_t dstate, mss_dtype io_dtype, uint32_t flags, void* hip_stream) {
  if (!h || !u || !delta || !A || !B || !C || !y) return MSS_ERR_NULL;
  if (!dtype_ok(io_dtype)) return MSS_ERR_DTYPE;
  if (batch <= 0 || dim <= 0 || dstate <= 0) return MSS_ERR_SHAPE;
  // At most 2^28 rows: 8 threads per row above 64 states keeps the grid below
  // 2^31 work-items, and every state offset below 2^35 elements.
  if (batch > (int64_t{1} << 28) || dim > (int64_t{1} << 28) || batch * dim > (int64_t{1} << 28))
    return MSS_ERR_SHAPE;
  if (dstate > 128) return MSS_ERR_UNSUPPORTED;
  if (flags != 0) return MSS_ERR_UNSUPPORTED;
  const void* all[] = {h, u, delta, A, B, C, D, z, y};
  for (const void* p : all)
    if (p && !aligned16(p)) return MSS_ERR_ALIGN;
  const size_t es = elem_size(io_dtype);
  const size_t nbd = (size_t)batch * dim;
  const size_t nstate = nbd * dstate * sizeof(float);
  const void* ins[] = {u, delta, A, B, C, D, z};
  const size_t in_bytes[] = {nbd * es, nbd * es, (size_t)dim * dstate * 4, (size_t)batch * dstate * es,
                             (size_t)batch * dstate * es, (size_t)dim * 4, nbd * es};
  if (!output_clear(h, nstate, ins, in_bytes, 7)) return MSS_ERR_ALIAS;
  if (!output_clear(y, nbd * es, ins, in_bytes, 7)) return MSS_ERR_ALIAS;
  if (overlaps(range_of(y, nbd * es), range_of(h, nstate))) return MSS_ERR_ALIAS;

  mss::UpdateParams p;
  p.h = h;
  p.u = u;
  p.delta = delta;
  p.A = A;
  p.B = B;
  p.C = C;
  p.D = D;
  p.z = z;
  p.y = y;
  p.batch = batch;
  p.dim = dim;
  p.dstate = dstate;
  p.bf16 = io_dtype == MSS_BF16;
  return hip_status(mss::launch_state_update(p, static_cast<hipStream_t>(hip_stream)));
}

// ---------------------------------------------------------- Mamba-3 update
mss_status mss_mamba3_state_update(float* h, const void* x, const void* x_prev, const float* delta, const float* A,
                                   const float* theta, const void* B, const void* B_prev, const void* C,
                                   const float* D, const void* z, void* y, int64_t batch, int64_t nheads,
                                   int64_t headdim, int64_t ngroups, int64_t dstate, int64_t rank,
                                   mss_dtype io_dtype, uint32_t flags, void* hip_stream) {
  if (!h || !x || !delta || !A || !B || !C || !y) return MSS_ERR_NULL;
  if ((x_prev == nullptr) != (B_prev == nullptr)) return MSS_ERR_NULL;
  const bool cplx = (flags & MSS_FLAG_COMPLEX_STATE) != 0;
  if (cplx && !theta) return MSS_ERR_NULL;
  if (!dtype_ok(io_dtype)) return MSS_ERR_DTYPE;
  if (batch <= 0 || nheads <= 0 || headdim <= 0 || ngroups <= 0 || dstate <= 0 || rank <= 0) return MSS_ERR_SHAPE;
  // Grid (headdim/16, nheads, batch); state offsets within 2^40 floats.
  if (batch > 65535 || nheads > 65535 || batch * nheads * headdim > (int64_t{1} << 28)) return MSS_ERR_SHAPE;
  if (flags & ~MSS_FLAG_COMPLEX_STATE) return MSS_ERR_UNSUPPORTED;
  if (headdim % 16 != 0 || headdim > 4096 || !(dstate == 64 || dstate == 128 || dstate == 256) || rank > 8 ||
      nheads % ngroups != 0)
    return MSS_ERR_UNSUPPORTED;
  const void* all[] = {h, delta, A, theta, D};
  for (const void* p : all)
    if (p && !aligned16(p)) return MSS_ERR_ALIGN;
  const size_t es = elem_size(io_dtype);
  const size_t nx = (size_t)batch * nheads * rank * headdim * es;
  const size_t nbc = (size_t)batch * ngroups * rank * dstate * es;
  const size_t nstate = (size_t)batch * nheads * headdim * dstate * sizeof(float) * (cplx ? 2 : 1);
  const void* ins[] = {x, x_prev, delta, A, theta, B, B_prev, C, D, z};
  const size_t in_bytes[] = {nx, nx, (size_t)batch * nheads * 4, (size_t)nheads * 4,
                             (size_t)nheads * dstate * 4, nbc, nbc, nbc, (size_t)nheads * 4, nx};
  if (!output_clear(h, nstate, ins, in_bytes, 10)) return MSS_ERR_ALIAS;
  if (!output_clear(y, nx, ins, in_bytes, 10)) return MSS_ERR_ALIAS;
  if (overlaps(range_of(y, nx), range_of(h, nstate))) return MSS_ERR_ALIAS;

  mss::Mamba3Params p;
  p.h = h;
  p.x = x;
  p.x_prev = x_prev;
  p.delta = delta;
  p.A = A;
  p.theta = cplx ? theta : nullptr;
  p.B = B;
  p.B_prev = B_prev;
  p.C = C;
  p.D = D;
  p.z = z;
  p.y = y;
  p.batch = batch;
  p.nheads = nheads;
  p.headdim = headdim;
  p.ngroups = ngroups;
  p.dstate = dstate;
  p.rank = rank;
  p.bf16 = io_dtype == MSS_BF16;
  return hip_status(mss::launch_mamba3_step(p, static_cast<hipStream_t>(hip_stream)));
}

// ----------------------------------------------------------------------- SSD
static mss_status ssd_check_shape(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                  int64_t ngroups, int64_t dstate, int64_t chunk, mss_dtype t) {
  if (!dtype_ok(t)) return MSS_ERR_DTYPE;
  if (batch <= 0 || seqlen <= 0 || nheads <= 0 || headdim <= 0 || ngroups <= 0 || dstate <= 0 || chunk <= 0)
    return MSS_ERR_SHAPE;
  // Byte offsets inside one batch entry of y (fp32) and of B, C must fit 32
  // bits, with every descriptor at most 2^32 - 256 bytes (the kernels' "no
  // element" offset lies past it).
  if (seqlen * nheads * headdim > (int64_t{1} << 30) - 64 || seqlen * ngroups * dstate >= (int64_t{1} << 30) ||
      batch > 65535 || nheads > 65535)
    return MSS_ERR_SHAPE;
  if (t != MSS_BF16) return MSS_ERR_UNSUPPORTED;
  if (!(headdim == 64 || headdim == 128) || dstate % 16 != 0 || dstate > 256 ||
      !(chunk == 64 || chunk == 128 || chunk == 256))
    return MSS_ERR_UNSUPPORTED;
  // Grids: at most 2 * (chunks x 64-row head slices x batch) workgroups of
  // 512 threads, below 2^32 work-items.
  if (((seqlen + chunk - 1) / chunk) * nheads * (headdim / 64) * batch >= (int64_t{1} << 22)) return MSS_ERR_SHAPE;
  if (nheads % ngroups != 0) return MSS_ERR_UNSUPPORTED;
  return MSS_OK;
}

size_t mss_ssd_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups,
                              int64_t dstate, int64_t chunk, mss_dtype in_dtype) {
  if (ssd_check_shape(batch, seqlen, nheads, headdim, ngroups, dstate, chunk, in_dtype) != MSS_OK) return 0;
  return mss::ssd_workspace_bytes(batch, seqlen, nheads, headdim, ngroups, dstate, chunk);
}

mss_status mss_ssd_chunk_fwd(const void* x, const float* delta, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* h0, float* y, float* chunk_states,
                             float* h_last, int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                             int64_t ngroups, int64_t dstate, int64_t chunk, mss_dtype in_dtype, uint32_t flags,
                             void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!x || !delta || !A || !B || !C || !y) return MSS_ERR_NULL;
  mss_status st = ssd_check_shape(batch, seqlen, nheads, headdim, ngroups, dstate, chunk, in_dtype);
  if (st != MSS_OK) return st;
  if (flags != 0) return MSS_ERR_UNSUPPORTED;
  const void* all[] = {x, delta, A, B, C, D, z, h0, y, chunk_states, h_last, workspace};
  for (const void* p : all)
    if (p && !aligned16(p)) return MSS_ERR_ALIGN;
  const size_t need = mss::ssd_workspace_bytes(batch, seqlen, nheads, headdim, ngroups, dstate, chunk);
  if (!workspace || workspace_bytes < need) return MSS_ERR_WORKSPACE;

  const size_t es = elem_size(in_dtype);
  const size_t nx = (size_t)batch * seqlen * nheads * headdim;
  const size_t nbc = (size_t)batch * seqlen * ngroups * dstate;
  const size_t nstate = (size_t)batch * nheads * headdim * dstate * sizeof(float);
  const size_t nchunks = (size_t)((seqlen + chunk - 1) / chunk);
  const void* ins[] = {x, delta, A, B, C, D, z, h0, workspace};
  const size_t in_bytes[] = {nx * es, (size_t)batch * seqlen * nheads * 4, (size_t)nheads * 4, nbc * es,
                             nbc * es, (size_t)nheads * 4, nx * es, nstate, need};
  const void* outs[] = {y, chunk_states, h_last};
  const size_t out_bytes[] = {nx * 4, nstate * nchunks, nstate};
  for (int i = 0; i < 3; ++i) {
    if (!output_clear(outs[i], out_bytes[i], ins, in_bytes, 9)) return MSS_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (outs[i] && outs[j] && overlaps(range_of(outs[i], out_bytes[i]), range_of(outs[j], out_bytes[j])))
        return MSS_ERR_ALIAS;
  }

  mss::SSDParams p;
  p.x = x;
  p.delta = delta;
  p.A = A;
  p.B = B;
  p.C = C;
  p.D = D;
  p.z = z;
  p.h0 = h0;
  p.y = y;
  p.chunk_states = chunk_states;
  p.h_last = h_last;
  p.batch = batch;
  p.seqlen = seqlen;
  p.nheads = nheads;
  p.headdim = headdim;
  p.ngroups = ngroups;
  p.dstate = dstate;
  p.chunk = chunk;
  p.workspace = workspace;
  return hip_status(mss::launch_ssd(p, static_cast<hipStream_t>(hip_stream)));
}


// The forward's limits with chunk 64 (d_state up to 256).  Up to 128 states
// one pass takes them all; above, two halves run one after the other.
static mss_status ssd_bwd_check_shape(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                      int64_t ngroups, int64_t dstate, mss_dtype t) {
  return ssd_check_shape(batch, seqlen, nheads, headdim, ngroups, dstate, 64, t);
}

static size_t ssd_bwd_need(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups,
                           int64_t dstate) {
  return dstate > 128 ? mss::ssd_bwd_halves_workspace_bytes(batch, seqlen, nheads, headdim, ngroups)
                      : mss::ssd_bwd_workspace_bytes(batch, seqlen, nheads, headdim, ngroups, dstate);
}

size_t mss_ssd_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                  int64_t ngroups, int64_t dstate, mss_dtype in_dtype) {
  if (ssd_bwd_check_shape(batch, seqlen, nheads, headdim, ngroups, dstate, in_dtype) != MSS_OK) return 0;
  return ssd_bwd_need(batch, seqlen, nheads, headdim, ngroups, dstate);
}

mss_status mss_ssd_chunk_bwd(const void* x, const float* delta, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* h0, const float* dy, const float* dh_last,
                             float* dx, float* ddelta, float* dA, float* dB, float* dC, float* dD, float* dz,
                             float* dh0, int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                             int64_t ngroups, int64_t dstate, mss_dtype in_dtype, uint32_t flags, void* workspace,
                             size_t workspace_bytes, void* hip_stream) {
  if (!x || !delta || !A || !B || !C || !dy || !dx || !ddelta || !dA || !dB || !dC) return MSS_ERR_NULL;
  if ((z == nullptr) != (dz == nullptr)) return MSS_ERR_NULL;
  mss_status st = ssd_bwd_check_shape(batch, seqlen, nheads, headdim, ngroups, dstate, in_dtype);
  if (st != MSS_OK) return st;
  if (flags != 0) return MSS_ERR_UNSUPPORTED;
  const void* all[] = {x, delta, A, B, C, D, z, h0, dy, dh_last, dx, ddelta, dA, dB, dC, dD, dz, dh0, workspace};
  for (const void* p : all)
    if (p && !aligned16(p)) return MSS_ERR_ALIGN;
  const size_t need = ssd_bwd_need(batch, seqlen, nheads, headdim, ngroups, dstate);
  if (!workspace || workspace_bytes < need) return MSS_ERR_WORKSPACE;

  const size_t es = elem_size(in_dtype);
  const size_t nx = (size_t)batch * seqlen * nheads * headdim;
  const size_t nbc = (size_t)batch * seqlen * ngroups * dstate;
  const size_t nstate = (size_t)batch * nheads * headdim * dstate * sizeof(float);
  const size_t ndl = (size_t)batch * seqlen * nheads * 4;
  const void* ins[] = {x, delta, A, B, C, D, z, h0, dy, dh_last, workspace};
  const size_t in_bytes[] = {nx * es, ndl, (size_t)nheads * 4, nbc * es, nbc * es, (size_t)nheads * 4, nx * es,
                             nstate, nx * 4, nstate, need};
  const void* outs[] = {dx, ddelta, dA, dB, dC, dD, dz, dh0};
  const size_t out_bytes[] = {nx * 4, ndl, (size_t)nheads * 4, nbc * 4, nbc * 4, (size_t)nheads * 4, nx * 4, nstate};
  for (int i = 0; i < 8; ++i) {
    if (!output_clear(outs[i], out_bytes[i], ins, in_bytes, 11)) return MSS_ERR_ALIAS;
    for (int j = i + 1; j < 8; ++j)
      if (outs[i] && outs[j] && overlaps(range_of(outs[i], out_bytes[i]), range_of(outs[j], out_bytes[j])))
        return MSS_ERR_ALIAS;
  }

  mss::SSDBwdParams p;
  p.x = x;
  p.delta = delta;
  p.A = A;
  p.B = B;
  p.C = C;
  p.D = D;
  p.z = z;
  p.h0 = h0;
  p.dy = dy;
  p.dh_last = dh_last;
  p.dx = dx;
  p.ddelta = ddelta;
  p.dA = dA;
  p.dB = dB;
  p.dC = dC;
  p.dD = dD;
  p.dz = dz;
  p.dh0 = dh0;
  p.batch = batch;
  p.seqlen = seqlen;
  p.nheads = nheads;
  p.headdim = headdim;
  p.ngroups = ngroups;
  p.dstate = dstate;
  p.workspace = workspace;
  if (dstate > 128) return hip_status(mss::launch_ssd_bwd_halves(p, static_cast<hipStream_t>(hip_stream)));
  return hip_status(mss::launch_ssd_bwd(p, static_cast<hipStream_t>(hip_stream)));
}

}  // extern "C"
