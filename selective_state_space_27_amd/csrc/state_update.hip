// Single-token state update (generation step) for gfx950.
//
// One step of the selective-scan recurrence with the state carried between
// calls ("Mamba-1/2/3 visual guide", section 2 figure: one-token generation
// uses the recurrent update of the same model; section 1: only the fixed-size
// state is carried).  Per (b, d):
//   h[n] <- exp(delta*A[d,n]) * h[n] + delta*B[b,n]*u ;  y = (C.h + D*u) * silu(z)
//
// The step is a pure stream over the fp32 state (read once, written once), so
// the kernel is laid out for HBM: 4 consecutive lanes own one channel's state
// row, each lane a contiguous slice of SPL states, so one wave instruction
// touches one contiguous span of the state (1 KB for N = 16).  The partial
// readouts of the 4 lanes are combined with a fixed butterfly (bitwise
// deterministic).  Decays use one hardware exp per state: the step is bound by
// the state stream, not by arithmetic.
#include "common.hpp"
#include "launch.hpp"

namespace mss {
namespace {

constexpr int kLanesPerChannel = 4;

template <bool BF16>
__device__ __forceinline__ float load_io(const void* p, size_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

template <bool BF16, int SPL>
__global__ void __launch_bounds__(256) state_update_kernel(float* __restrict__ h, const void* __restrict__ u,
                                                           const void* __restrict__ delta, const float* __restrict__ A,
                                                           const void* __restrict__ B, const void* __restrict__ C,
                                                           const float* __restrict__ D, const void* __restrict__ z,
                                                           void* __restrict__ y, int batch, int dim, int N) {
  const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t bd = gid / kLanesPerChannel;       // (b, d) pair
  const int q = (int)(gid % kLanesPerChannel);    // slice of the state row
  const bool active = bd < (size_t)batch * dim;
  const size_t bds = active ? bd : 0;
  const int b = (int)(bds / dim);
  const int d = (int)(bds % dim);
  const int n0 = q * SPL;

  const float uu = load_io<BF16>(u, bds);
  const float dl = load_io<BF16>(delta, bds);
  const float du = dl * uu;

  float hv[SPL], av[SPL], bv[SPL], cv[SPL];
  float* hrow = h + bds * N;
  const float* arow = A + (size_t)d * N;
  const bool full = (N == kLanesPerChannel * SPL);
  if (full && SPL % 4 == 0) {
#pragma unroll
    for (int j = 0; j < SPL; j += 4) {
      const float4 t = *reinterpret_cast<const float4*>(hrow + n0 + j);
      const float4 s = *reinterpret_cast<const float4*>(arow + n0 + j);
      hv[j] = t.x; hv[j + 1] = t.y; hv[j + 2] = t.z; hv[j + 3] = t.w;
      av[j] = s.x; av[j + 1] = s.y; av[j + 2] = s.z; av[j + 3] = s.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
      const bool ok = n0 + j < N;
      hv[j] = ok ? hrow[n0 + j] : 0.f;
      av[j] = ok ? arow[n0 + j] : 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    const bool ok = n0 + j < N;
    bv[j] = ok ? load_io<BF16>(B, (size_t)b * N + n0 + j) : 0.f;
    cv[j] = ok ? load_io<BF16>(C, (size_t)b * N + n0 + j) : 0.f;
  }

  float p = 0.f;
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    const float dec = exp2_fast(dl * av[j] * kLog2e);
    hv[j] = __builtin_fmaf(dec, hv[j], du * bv[j]);
    p = __builtin_fmaf(cv[j], hv[j], p);
  }
  // Fixed-order butterfly over the 4 lanes of the channel.
  p += __shfl_xor(p, 1, kLanesPerChannel);
  p += __shfl_xor(p, 2, kLanesPerChannel);

  if (!active) return;
  if (full && SPL % 4 == 0) {
#pragma unroll
    for (int j = 0; j < SPL; j += 4)
      *reinterpret_cast<float4*>(hrow + n0 + j) = make_float4(hv[j], hv[j + 1], hv[j + 2], hv[j + 3]);
  } else {
#pragma unroll
    for (int j = 0; j < SPL; ++j)
      if (n0 + j < N) hrow[n0 + j] = hv[j];
  }
  if (q == 0) {
    float out = __builtin_fmaf(D != nullptr ? D[d] : 0.f, uu, p);
    if (z != nullptr) out *= silu(load_io<BF16>(z, bds));
    if constexpr (BF16) static_cast<uint16_t*>(y)[bds] = f32_to_bf16(out);
    else static_cast<float*>(y)[bds] = out;
  }
}

template <bool BF16, int SPL>
hipError_t launch_typed(const UpdateParams& p, hipStream_t stream) {
  const size_t threads = (size_t)p.batch * p.dim * kLanesPerChannel;
  const unsigned grid = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL((state_update_kernel<BF16, SPL>), dim3(grid), dim3(256), 0, stream, p.h, p.u, p.delta, p.A,
                     p.B, p.C, p.D, p.z, p.y, (int)p.batch, (int)p.dim, (int)p.dstate);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const UpdateParams& p, hipStream_t stream) {
  const int64_t n = p.dstate;
  if (n <= 4) return launch_typed<BF16, 1>(p, stream);
  if (n <= 8) return launch_typed<BF16, 2>(p, stream);
  if (n <= 16) return launch_typed<BF16, 4>(p, stream);
  if (n <= 32) return launch_typed<BF16, 8>(p, stream);
  return launch_typed<BF16, 16>(p, stream);
}

}  // namespace

hipError_t launch_state_update(const UpdateParams& p, hipStream_t stream) {
  return p.bf16 ? launch_dtype<true>(p, stream) : launch_dtype<false>(p, stream);
}

}  // namespace mss
