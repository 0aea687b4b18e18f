// Backward of the SSD layer for d_state 129..256, by two halves of the states.
//
// Within a head every state column evolves on its own under the head's
// scalar decay ("Mamba-1/2/3 visual guide", section 3: A is a scalar times
// the identity per head), and the output couples the columns only through
// the readout C.h.  So the gradient splits over the first 128 states and the
// rest, each half handled by the d_state <= 128 backward (ssd_bwd.hip) on
// the half's B/C columns and h0/dh_last columns:
//   - dB, dC, dh0 of a state come from its half;
//   - dx, ddelta, dA and dz are sums over states, so they are the sums of the
//     two halves' values; the skip term D (D x in the output and in dx, and
//     dD) is the first half's only.
// Every gradient of the SSD backward is fp32: the first half writes dx,
// ddelta, dA and dz in place and the second half's are added to them.
//
// Workspace: a 256-byte head (word 0: the call's status, word 1: the halves'
// status words or-ed together), one d_state-128 backward workspace reused by
// both halves, then the buffers below.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace mss {
namespace {

constexpr int kHalf = 128;
constexpr size_t kMaxHalvesGrid = 16384;

inline unsigned halves_grid(size_t items) {
  return (unsigned)std::max<size_t>(1, std::min<size_t>((items + 255) / 256, kMaxHalvesGrid));
}
inline size_t al256h(size_t x) { return (x + 255) & ~(size_t)255; }

// Columns [n0, n0+nh) of rows of length N: dst[r*nh + j] = src[r*N + n0 + j]
// (ES-byte elements: 2 for the bf16 B and C, 4 for the fp32 states).
template <typename T>
__global__ void __launch_bounds__(256) half_gather(const T* __restrict__ src, T* __restrict__ dst, size_t rows, int N,
                                                   int n0, int nh) {
  const size_t total = rows * (size_t)nh;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const size_t r = i / (size_t)nh, j = i % (size_t)nh;
    dst[i] = src[r * (size_t)N + (size_t)n0 + j];
  }
}

// The inverse placement: dst[r*N + n0 + j] = src[r*nh + j].
__global__ void __launch_bounds__(256) half_scatter(const float* __restrict__ src, float* __restrict__ dst,
                                                    size_t rows, int N, int n0, int nh) {
  const size_t total = rows * (size_t)nh;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const size_t r = i / (size_t)nh, j = i % (size_t)nh;
    dst[r * (size_t)N + (size_t)n0 + j] = src[i];
  }
}

// dst[i] += src[i], four elements per thread and step (one 16-byte access
// each when whole: the bases are 16-byte aligned and i a multiple of 4).
__global__ void __launch_bounds__(256) half_add(const float* __restrict__ src, float* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x * 4;
  for (size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n) {
      const float4 a = *reinterpret_cast<const float4*>(dst + i), b = *reinterpret_cast<const float4*>(src + i);
      *reinterpret_cast<float4*>(dst + i) = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
    } else {
      for (size_t k = i; k < n; ++k) dst[k] += src[k];
    }
  }
}

// Status words: mode 0 clears the head, 1 ors a half's word into word 1,
// 2 publishes word 1 as the call's status (word 0).
__global__ void half_status(int* __restrict__ head, const int* __restrict__ half_word, int mode) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  if (mode == 0) {
    head[0] = 0;
    head[1] = 0;
  } else if (mode == 1) {
    head[1] |= *half_word;
  } else {
    head[0] = head[1];
  }
}

struct HalvesLayout {
  size_t head, half_ws, B, C, h0, dhl, dx, ddelta, dA, dz, dB, dC, dh0, total;
};

HalvesLayout halves_layout(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups) {
  const size_t nx = (size_t)batch * seqlen * nheads * headdim;
  const size_t nbc = (size_t)batch * seqlen * ngroups * kHalf;
  const size_t nst = (size_t)batch * nheads * headdim * kHalf;
  HalvesLayout l;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += al256h(bytes);
    return at;
  };
  l.head = take(256);
  l.half_ws = take(ssd_bwd_workspace_bytes(batch, seqlen, nheads, headdim, ngroups, kHalf));
  l.B = take(nbc * 2);
  l.C = take(nbc * 2);
  l.h0 = take(nst * 4);
  l.dhl = take(nst * 4);
  l.dx = take(nx * 4);
  l.ddelta = take((size_t)batch * seqlen * nheads * 4);
  l.dA = take((size_t)nheads * 4);
  l.dz = take(nx * 4);
  l.dB = take(nbc * 4);
  l.dC = take(nbc * 4);
  l.dh0 = take(nst * 4);
  l.total = o;
  return l;
}

}  // namespace

size_t ssd_bwd_halves_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                      int64_t ngroups) {
  return halves_layout(batch, seqlen, nheads, headdim, ngroups).total;
}

hipError_t launch_ssd_bwd_halves(const SSDBwdParams& p, hipStream_t stream) {
  const HalvesLayout l = halves_layout(p.batch, p.seqlen, p.nheads, p.headdim, p.ngroups);
  char* ws = static_cast<char*>(p.workspace);
  auto fp = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  auto hp = [&](size_t off) { return reinterpret_cast<uint16_t*>(ws + off); };
  int* head = reinterpret_cast<int*>(ws + l.head);
  const int N = (int)p.dstate;
  const size_t bc_rows = (size_t)p.batch * p.seqlen * p.ngroups;
  const size_t st_rows = (size_t)p.batch * p.nheads * p.headdim;
  const size_t nx = (size_t)p.batch * p.seqlen * p.nheads * p.headdim;
  const size_t ndl = (size_t)p.batch * p.seqlen * p.nheads;
  hipError_t err = hipSuccess;
  auto check = [&]() {
    err = hipGetLastError();
    return err == hipSuccess;
  };

  hipLaunchKernelGGL(half_status, dim3(1), dim3(64), 0, stream, head, head, 0);
  for (int h = 0; h < 2; ++h) {
    const int n0 = h * kHalf, nh = std::min(kHalf, N - n0);
    const auto* B = static_cast<const uint16_t*>(p.B);
    const auto* C = static_cast<const uint16_t*>(p.C);
    hipLaunchKernelGGL(half_gather<uint16_t>, dim3(halves_grid(bc_rows * nh)), dim3(256), 0, stream, B, hp(l.B),
                       bc_rows, N, n0, nh);
    hipLaunchKernelGGL(half_gather<uint16_t>, dim3(halves_grid(bc_rows * nh)), dim3(256), 0, stream, C, hp(l.C),
                       bc_rows, N, n0, nh);
    if (p.h0)
      hipLaunchKernelGGL(half_gather<float>, dim3(halves_grid(st_rows * nh)), dim3(256), 0, stream, p.h0, fp(l.h0),
                         st_rows, N, n0, nh);
    if (p.dh_last)
      hipLaunchKernelGGL(half_gather<float>, dim3(halves_grid(st_rows * nh)), dim3(256), 0, stream, p.dh_last,
                         fp(l.dhl), st_rows, N, n0, nh);
    if (!check()) return err;

    SSDBwdParams q = p;
    q.B = hp(l.B);
    q.C = hp(l.C);
    q.h0 = p.h0 ? fp(l.h0) : nullptr;
    q.dh_last = p.dh_last ? fp(l.dhl) : nullptr;
    q.D = h == 0 ? p.D : nullptr;  // the skip term belongs to one half
    q.dD = h == 0 ? p.dD : nullptr;
    q.dstate = nh;
    q.workspace = ws + l.half_ws;
    if (h == 1) {  // the second half's sums go to scratch, then are added
      q.dx = fp(l.dx);
      q.ddelta = fp(l.ddelta);
      q.dA = fp(l.dA);
      q.dz = p.dz ? fp(l.dz) : nullptr;
    }
    q.dB = fp(l.dB);
    q.dC = fp(l.dC);
    q.dh0 = p.dh0 ? fp(l.dh0) : nullptr;
    err = launch_ssd_bwd(q, stream);
    if (err != hipSuccess) return err;

    hipLaunchKernelGGL(half_status, dim3(1), dim3(64), 0, stream, head, reinterpret_cast<const int*>(ws + l.half_ws),
                       1);
    hipLaunchKernelGGL(half_scatter, dim3(halves_grid(bc_rows * nh)), dim3(256), 0, stream, fp(l.dB), p.dB, bc_rows, N,
                       n0, nh);
    hipLaunchKernelGGL(half_scatter, dim3(halves_grid(bc_rows * nh)), dim3(256), 0, stream, fp(l.dC), p.dC, bc_rows, N,
                       n0, nh);
    if (p.dh0)
      hipLaunchKernelGGL(half_scatter, dim3(halves_grid(st_rows * nh)), dim3(256), 0, stream, fp(l.dh0), p.dh0,
                         st_rows, N, n0, nh);
    if (h == 1) {
      hipLaunchKernelGGL(half_add, dim3(halves_grid((nx + 3) / 4)), dim3(256), 0, stream, fp(l.dx), p.dx, nx);
      hipLaunchKernelGGL(half_add, dim3(halves_grid((ndl + 3) / 4)), dim3(256), 0, stream, fp(l.ddelta), p.ddelta, ndl);
      hipLaunchKernelGGL(half_add, dim3(1), dim3(256), 0, stream, fp(l.dA), p.dA, (size_t)p.nheads);
      if (p.dz) hipLaunchKernelGGL(half_add, dim3(halves_grid((nx + 3) / 4)), dim3(256), 0, stream, fp(l.dz), p.dz, nx);
    }
    if (!check()) return err;
  }
  hipLaunchKernelGGL(half_status, dim3(1), dim3(64), 0, stream, head, head, 2);
  check();
  return err;
}

}  // namespace mss
