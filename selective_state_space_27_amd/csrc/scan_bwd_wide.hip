// Backward of the selective scan for d_state 33..128, by slices of the states.
//
// The states of a channel evolve independently of one another: state n's
// recurrence reads only A[d,n], B[.,n], delta and u ("Mamba (deep learning)",
// state-space paragraph; "Mamba-1/2/3 visual guide", section 1 equation), and
// the output couples them only through the readout sum C.h.  So the gradient
// splits over slices of at most 32 states, each handled by the d_state <= 32
// backward (scan_bwd.hip) on the slice's A columns, B/C rows, h0 and dh_last
// columns:
//   - dA, dB, dC, dh0 of a state come from its own slice;
//   - du, ddelta and dz are sums over states (du = sum_n dh delta B + D dout,
//     ddelta = sum_n dh (h_prev a A + B u), dz = dy out silu'(z) with out the
//     ungated output, linear in the readout), so they are the sums of the
//     slices' values, the skip term D (D u in out, D dout in du) taken by
//     slice 0 only, whose dD is the call's.
// The slices run in fp32 (bf16 inputs are widened exactly once), their du,
// ddelta and dz are summed in fp32 in slice order, and the sums are rounded to
// the I/O type once at the end, as are dB and dC.
//
// Workspace: a 256-byte head (word 0: the call's status, word 1: the slices'
// status words or-ed together), one d_state-32 backward workspace reused by
// every slice, then the fp32 buffers below.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace mss {
namespace {

constexpr int kSlice = 32;  // states per slice: the d_state <= 32 backward's limit
constexpr size_t kMaxWideGrid = 16384;

inline unsigned wide_grid(size_t items) {
  return (unsigned)std::max<size_t>(1, std::min<size_t>((items + 255) / 256, kMaxWideGrid));
}
// The flat passes over [b, d, L] take four elements per thread and step.
inline unsigned wide_grid4(size_t items) { return wide_grid((items + 3) / 4); }
inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

__device__ __forceinline__ float ld_any(const void* p, size_t i, bool bf16) {
  return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

// Four consecutive elements i..i+3 (k < n of them; n = 4 is one 8-byte bf16
// or 16-byte fp32 access, i being a multiple of 4 from a 16-byte-aligned
// base), read as fp32 or written narrowed to the output type (bf16 round to
// nearest even).  One element per thread and access left these passes far
// below the HBM rate.
__device__ __forceinline__ void wide_ld4(const void* p, size_t i, int n, bool bf16, float (&v)[4]) {
  if (n == 4 && bf16) {
    const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    v[0] = __uint_as_float(q.x << 16);
    v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16);
    v[3] = __uint_as_float(q.y & 0xffff0000u);
  } else if (n == 4) {
    const float4 q = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    v[0] = q.x;
    v[1] = q.y;
    v[2] = q.z;
    v[3] = q.w;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = k < n ? ld_any(p, i + k, bf16) : 0.f;
  }
}
__device__ __forceinline__ void wide_st4(void* p, size_t i, int n, bool bf16, const float (&v)[4]) {
  if (n == 4 && bf16) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i) = make_uint2(pack_bf16x2(v[0], v[1]),
                                                                          pack_bf16x2(v[2], v[3]));
  } else if (n == 4) {
    *reinterpret_cast<float4*>(static_cast<float*>(p) + i) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k >= n) break;
      if (bf16) static_cast<uint16_t*>(p)[i + k] = f32_to_bf16(v[k]);
      else static_cast<float*>(p)[i + k] = v[k];
    }
  }
}

// dst[i] = src[i] widened to fp32.
__global__ void __launch_bounds__(256) wide_to_f32(const void* __restrict__ src, float* __restrict__ dst, size_t n,
                                                   int bf16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x * 4;
  for (size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    const int m = (int)std::min<size_t>(4, n - i);
    float v[4];
    wide_ld4(src, i, m, bf16 != 0, v);
    wide_st4(dst, i, m, false, v);
  }
}

// Columns [n0, n0+ns) of rows of length N: dst[r*ns + j] = src[r*N + n0 + j]
// (A and the [b, d, N] states), or rows [n0, n0+ns) of [outer][N][L] planes
// (B, C): dst[(o*ns + j)*L + l] = src[(o*N + n0 + j)*L + l].  Widened to fp32.
__global__ void __launch_bounds__(256) wide_gather(const void* __restrict__ src, float* __restrict__ dst,
                                                   size_t outer, int N, int n0, int ns, size_t inner, int bf16) {
  const size_t total = outer * (size_t)ns * inner;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const size_t in = i % inner;
    const size_t j = (i / inner) % (size_t)ns;
    const size_t o = i / (inner * (size_t)ns);
    dst[i] = ld_any(src, (o * (size_t)N + (size_t)n0 + j) * inner + in, bf16);
  }
}

// The inverse placement of wide_gather, narrowed to the output type (bf16
// round to nearest even).
__global__ void __launch_bounds__(256) wide_scatter(const float* __restrict__ src, void* __restrict__ dst,
                                                    size_t outer, int N, int n0, int ns, size_t inner, int bf16) {
  const size_t total = outer * (size_t)ns * inner;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const size_t in = i % inner;
    const size_t j = (i / inner) % (size_t)ns;
    const size_t o = i / (inner * (size_t)ns);
    const size_t k = (o * (size_t)N + (size_t)n0 + j) * inner + in;
    if (bf16) static_cast<uint16_t*>(dst)[k] = f32_to_bf16(src[i]);
    else static_cast<float*>(dst)[k] = src[i];
  }
}

// acc = src (first slice) or acc + src; up to three arrays per launch.
__global__ void __launch_bounds__(256) wide_accumulate(const float* __restrict__ s0, float* __restrict__ a0,
                                                       const float* __restrict__ s1, float* __restrict__ a1,
                                                       const float* __restrict__ s2, float* __restrict__ a2, size_t n,
                                                       int first) {
  const size_t stride = (size_t)gridDim.x * blockDim.x * 4;
  const float* src[3] = {s0, s1, s2};
  float* acc[3] = {a0, a1, a2};
  for (size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    const int m = (int)std::min<size_t>(4, n - i);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      if (src[q] == nullptr) continue;
      float v[4];
      wide_ld4(src[q], i, m, false, v);
      if (!first) {
        float a[4];
        wide_ld4(acc[q], i, m, false, a);
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = a[k] + v[k];
      }
      wide_st4(acc[q], i, m, false, v);
    }
  }
}

// dst[i] = src[i] narrowed to the output type.
__global__ void __launch_bounds__(256) wide_from_f32(const float* __restrict__ src, void* __restrict__ dst, size_t n,
                                                     int bf16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x * 4;
  for (size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    const int m = (int)std::min<size_t>(4, n - i);
    float v[4];
    wide_ld4(src, i, m, false, v);
    wide_st4(dst, i, m, bf16 != 0, v);
  }
}

// Status words: mode 0 clears the head, 1 ors a slice's word into word 1,
// 2 publishes word 1 as the call's status (word 0).
__global__ void wide_status(int* __restrict__ head, const int* __restrict__ slice_word, int mode) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  if (mode == 0) {
    head[0] = 0;
    head[1] = 0;
  } else if (mode == 1) {
    head[1] |= *slice_word;
  } else {
    head[0] = head[1];
  }
}

struct WideLayout {
  size_t head, slice_ws, u, delta, dy, z, A, B, C, h0, dhl, du, ddelta, dz, dA, dB, dC, dh0, acc_du, acc_dd,
      acc_dz, total;
};

WideLayout wide_layout(int64_t batch, int64_t dim, int64_t seqlen) {
  const size_t bdl = (size_t)batch * dim * seqlen * sizeof(float);
  const size_t bnl = (size_t)batch * kSlice * seqlen * sizeof(float);
  const size_t dn = (size_t)dim * kSlice * sizeof(float);
  const size_t bdn = (size_t)batch * dim * kSlice * sizeof(float);
  WideLayout l;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += al256(bytes);
    return at;
  };
  l.head = take(256);
  l.slice_ws = take(scan_bwd_workspace_bytes(batch, dim, kSlice, seqlen));
  l.u = take(bdl);
  l.delta = take(bdl);
  l.dy = take(bdl);
  l.z = take(bdl);
  l.A = take(dn);
  l.B = take(bnl);
  l.C = take(bnl);
  l.h0 = take(bdn);
  l.dhl = take(bdn);
  l.du = take(bdl);
  l.ddelta = take(bdl);
  l.dz = take(bdl);
  l.dA = take(dn);
  l.dB = take(bnl);
  l.dC = take(bnl);
  l.dh0 = take(bdn);
  l.acc_du = take(bdl);
  l.acc_dd = take(bdl);
  l.acc_dz = take(bdl);
  l.total = o;
  return l;
}

}  // namespace

size_t scan_bwd_wide_workspace_bytes(int64_t batch, int64_t dim, int64_t seqlen) {
  return wide_layout(batch, dim, seqlen).total;
}

hipError_t launch_scan_bwd_wide(const ScanBwdParams& p, hipStream_t stream) {
  const ScanParams& f = p.fwd;
  const WideLayout l = wide_layout(f.batch, f.dim, f.seqlen);
  char* ws = static_cast<char*>(f.workspace);
  auto fp = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  int* head = reinterpret_cast<int*>(ws + l.head);
  const int bf16 = f.bf16 ? 1 : 0;
  const size_t bdl = (size_t)f.batch * f.dim * f.seqlen;
  const size_t bd = (size_t)f.batch * f.dim;
  const int N = (int)f.dstate;
  hipError_t err = hipSuccess;
  auto check = [&]() {
    err = hipGetLastError();
    return err == hipSuccess;
  };

  hipLaunchKernelGGL(wide_status, dim3(1), dim3(64), 0, stream, head, head, 0);
  // The [b, d, L] inputs in fp32 (bf16 widened; fp32 used as given).
  const float* u32 = static_cast<const float*>(f.u);
  const float* d32 = static_cast<const float*>(f.delta);
  const float* dy32 = static_cast<const float*>(p.dy);
  const float* z32 = static_cast<const float*>(f.z);
  if (bf16) {
    const void* src[4] = {f.u, f.delta, p.dy, f.z};
    float* dst[4] = {fp(l.u), fp(l.delta), fp(l.dy), fp(l.z)};
    for (int i = 0; i < 4; ++i) {
      if (src[i] == nullptr) continue;
      hipLaunchKernelGGL(wide_to_f32, dim3(wide_grid4(bdl)), dim3(256), 0, stream, src[i], dst[i], bdl, 1);
    }
    u32 = dst[0], d32 = dst[1], dy32 = dst[2], z32 = f.z ? dst[3] : nullptr;
  }
  if (!check()) return err;

  for (int n0 = 0, s = 0; n0 < N; n0 += kSlice, ++s) {
    const int ns = std::min(kSlice, N - n0);
    hipLaunchKernelGGL(wide_gather, dim3(wide_grid((size_t)f.dim * ns)), dim3(256), 0, stream,
                       static_cast<const void*>(f.A), fp(l.A), (size_t)f.dim, N, n0, ns, (size_t)1, 0);
    hipLaunchKernelGGL(wide_gather, dim3(wide_grid((size_t)f.batch * ns * f.seqlen)), dim3(256), 0, stream, f.B,
                       fp(l.B), (size_t)f.batch, N, n0, ns, (size_t)f.seqlen, bf16);
    hipLaunchKernelGGL(wide_gather, dim3(wide_grid((size_t)f.batch * ns * f.seqlen)), dim3(256), 0, stream, f.C,
                       fp(l.C), (size_t)f.batch, N, n0, ns, (size_t)f.seqlen, bf16);
    if (f.h0)
      hipLaunchKernelGGL(wide_gather, dim3(wide_grid(bd * ns)), dim3(256), 0, stream,
                         static_cast<const void*>(f.h0), fp(l.h0), bd, N, n0, ns, (size_t)1, 0);
    if (p.dh_last)
      hipLaunchKernelGGL(wide_gather, dim3(wide_grid(bd * ns)), dim3(256), 0, stream,
                         static_cast<const void*>(p.dh_last), fp(l.dhl), bd, N, n0, ns, (size_t)1, 0);
    if (!check()) return err;

    ScanBwdParams q;
    q.fwd = f;
    q.fwd.u = u32;
    q.fwd.delta = d32;
    q.fwd.A = fp(l.A);
    q.fwd.B = fp(l.B);
    q.fwd.C = fp(l.C);
    q.fwd.D = s == 0 ? f.D : nullptr;  // the skip term belongs to one slice
    q.fwd.z = z32;
    q.fwd.h0 = f.h0 ? fp(l.h0) : nullptr;
    q.fwd.y = nullptr;
    q.fwd.h_last = nullptr;
    q.fwd.dstate = ns;
    q.fwd.bf16 = false;
    q.fwd.workspace = ws + l.slice_ws;
    q.fwd.status = nullptr;
    q.dy = dy32;
    q.dh_last = p.dh_last ? fp(l.dhl) : nullptr;
    q.du = fp(l.du);
    q.ddelta = fp(l.ddelta);
    q.dA = fp(l.dA);
    q.dB = fp(l.dB);
    q.dC = fp(l.dC);
    q.dD = s == 0 ? p.dD : nullptr;
    q.dz = z32 ? fp(l.dz) : nullptr;
    q.dh0 = p.dh0 ? fp(l.dh0) : nullptr;
    err = launch_scan_bwd(q, stream);
    if (err != hipSuccess) return err;

    hipLaunchKernelGGL(wide_status, dim3(1), dim3(64), 0, stream, head, reinterpret_cast<const int*>(ws + l.slice_ws),
                       1);
    hipLaunchKernelGGL(wide_accumulate, dim3(wide_grid4(bdl)), dim3(256), 0, stream, fp(l.du), fp(l.acc_du),
                       fp(l.ddelta), fp(l.acc_dd), z32 ? fp(l.dz) : nullptr, fp(l.acc_dz), bdl, s == 0 ? 1 : 0);
    hipLaunchKernelGGL(wide_scatter, dim3(wide_grid((size_t)f.dim * ns)), dim3(256), 0, stream, fp(l.dA),
                       static_cast<void*>(p.dA), (size_t)f.dim, N, n0, ns, (size_t)1, 0);
    hipLaunchKernelGGL(wide_scatter, dim3(wide_grid((size_t)f.batch * ns * f.seqlen)), dim3(256), 0, stream,
                       fp(l.dB), p.dB, (size_t)f.batch, N, n0, ns, (size_t)f.seqlen, bf16);
    hipLaunchKernelGGL(wide_scatter, dim3(wide_grid((size_t)f.batch * ns * f.seqlen)), dim3(256), 0, stream,
                       fp(l.dC), p.dC, (size_t)f.batch, N, n0, ns, (size_t)f.seqlen, bf16);
    if (p.dh0)
      hipLaunchKernelGGL(wide_scatter, dim3(wide_grid(bd * ns)), dim3(256), 0, stream, fp(l.dh0),
                         static_cast<void*>(p.dh0), bd, N, n0, ns, (size_t)1, 0);
    if (!check()) return err;
  }

  hipLaunchKernelGGL(wide_from_f32, dim3(wide_grid4(bdl)), dim3(256), 0, stream, fp(l.acc_du), p.du, bdl, bf16);
  hipLaunchKernelGGL(wide_from_f32, dim3(wide_grid4(bdl)), dim3(256), 0, stream, fp(l.acc_dd), p.ddelta, bdl, bf16);
  if (z32) hipLaunchKernelGGL(wide_from_f32, dim3(wide_grid4(bdl)), dim3(256), 0, stream, fp(l.acc_dz), p.dz, bdl, bf16);
  hipLaunchKernelGGL(wide_status, dim3(1), dim3(64), 0, stream, head, head, 2);
  check();
  return err;
}

}  // namespace mss
