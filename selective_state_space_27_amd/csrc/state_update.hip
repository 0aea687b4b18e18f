// Single-token state update (generation step) for gfx950.
//
// One step of the selective-scan recurrence with the state carried between
// calls ("Mamba-1/2/3 visual guide", section 2 figure: one-token generation
// uses the recurrent update of the same model; section 1: only the fixed-size
// state is carried).  Per (b, d):
//   h[n] <- exp(delta*A[d,n]) * h[n] + delta*B[b,n]*u ;  y = (C.h + D*u) * silu(z)
//
// The step is a pure stream over the fp32 state (read once, written once), so
// the kernel is laid out for HBM: LPC consecutive lanes (4, or 8 for N > 64)
// own one channel's state row, each lane a contiguous slice of SPL states, so
// one wave instruction touches one contiguous span of the state (1 KB for
// N = 16).  Each thread handles kRows channel rows (two for N <= 64, one
// above) 64/LPC channels apart and issues every load of all of them before
// any arithmetic, so a wave keeps kRows such spans in flight (the step is
// bound by how many state bytes are in flight, not by arithmetic; two rows
// measured best at N = 16, more rows cost occupancy).  The new state is
// written with non-temporal stores.  The partial readouts of a channel's
// lanes are combined with a fixed butterfly (bitwise deterministic).  Decays
// use one hardware exp per state.
#include "common.hpp"
#include "launch.hpp"

namespace mss {
namespace {

// Channel rows per thread: two for N <= 64 (measured best there); one for the
// 8-lane rows above 64, whose 16 states per lane already fill the registers.
template <int LPC>
constexpr int rows_per_thread() { return LPC == 4 ? 2 : 1; }
constexpr int kThreadsSU = 256;

template <bool BF16>
__device__ __forceinline__ float load_io(const void* p, size_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

// SPL consecutive B (or C) values from n0 of batch row b: 4 at a time when
// the slices are whole and aligned (`fast`), else one by one with a bound.
template <bool BF16, int SPL>
__device__ __forceinline__ void load_vec(const void* p, size_t off, int n0, int N, bool fast, float* v) {
  if constexpr (SPL % 4 == 0) {
    if (fast) {
#pragma unroll
      for (int j = 0; j < SPL; j += 4) {
        if constexpr (BF16) {
          const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + off + j);
          v[j] = bf16_lo(w.x); v[j + 1] = bf16_hi(w.x); v[j + 2] = bf16_lo(w.y); v[j + 3] = bf16_hi(w.y);
        } else {
          const float4 w = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + off + j);
          v[j] = w.x; v[j + 1] = w.y; v[j + 2] = w.z; v[j + 3] = w.w;
        }
      }
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < SPL; ++j) v[j] = (n0 + j < N) ? load_io<BF16>(p, off + j) : 0.f;
}

template <bool BF16, int SPL, int LPC>
__global__ void __launch_bounds__(kThreadsSU) state_update_kernel(float* __restrict__ h, const void* __restrict__ u,
                                                                 const void* __restrict__ delta,
                                                                 const float* __restrict__ A,
                                                                 const void* __restrict__ B,
                                                                 const void* __restrict__ C,
                                                                 const float* __restrict__ D,
                                                                 const void* __restrict__ z, void* __restrict__ y,
                                                                 int batch, int dim, int N) {
  const size_t gid = (size_t)blockIdx.x * kThreadsSU + threadIdx.x;
  const int lane = threadIdx.x & 63;
  constexpr int kCh = 64 / LPC;  // channels per row set of a wave
  constexpr int kRows = rows_per_thread<LPC>();
  const int q = lane % LPC;       // slice of the state row
  const int n0 = q * SPL;
  // A wave covers kCh consecutive channels per row set and kRows row sets.
  const size_t row0 = (gid >> 6) * (kCh * kRows) + (size_t)(lane / LPC);
  const size_t nrows = (size_t)batch * dim;
  // Vector loads need whole aligned slices: N equal to LPC lanes * SPL.
  const bool full = (N == LPC * SPL) && (SPL % 4 == 0);
  const bool bc_fast = full && ((N * (BF16 ? 2 : 4)) % 8 == 0);

  float hv[kRows][SPL], av[kRows][SPL], bv[kRows][SPL], cv[kRows][SPL];
  float uu[kRows], dl[kRows], zz[kRows], dd[kRows];
  bool act[kRows];
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    const size_t bd = row0 + (size_t)k * kCh;
    act[k] = bd < nrows;
    const size_t bds = act[k] ? bd : 0;
    const int b = (int)(bds / dim);
    const int d = (int)(bds % dim);
    const float* hrow = h + bds * N;
    const float* arow = A + (size_t)d * N;
    if (full) {
#pragma unroll
      for (int j = 0; j < SPL; j += 4) {
        const float4 t = *reinterpret_cast<const float4*>(hrow + n0 + j);
        const float4 s = *reinterpret_cast<const float4*>(arow + n0 + j);
        hv[k][j] = t.x; hv[k][j + 1] = t.y; hv[k][j + 2] = t.z; hv[k][j + 3] = t.w;
        av[k][j] = s.x; av[k][j + 1] = s.y; av[k][j + 2] = s.z; av[k][j + 3] = s.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        const bool ok = n0 + j < N;
        hv[k][j] = ok ? hrow[n0 + j] : 0.f;
        av[k][j] = ok ? arow[n0 + j] : 0.f;
      }
    }
    load_vec<BF16, SPL>(B, (size_t)b * N + n0, n0, N, bc_fast, bv[k]);
    load_vec<BF16, SPL>(C, (size_t)b * N + n0, n0, N, bc_fast, cv[k]);
    uu[k] = load_io<BF16>(u, bds);
    dl[k] = load_io<BF16>(delta, bds);
    zz[k] = z != nullptr ? load_io<BF16>(z, bds) : 0.f;
    dd[k] = D != nullptr ? D[d] : 0.f;
  }

#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    const float du = dl[k] * uu[k];
    float p = 0.f;
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
      const float dec = exp2_fast(dl[k] * av[k][j] * kLog2e);
      hv[k][j] = __builtin_fmaf(dec, hv[k][j], du * bv[k][j]);
      p = __builtin_fmaf(cv[k][j], hv[k][j], p);
    }
    // Fixed-order butterfly over the LPC lanes of the channel.
#pragma unroll
    for (int m = 1; m < LPC; m <<= 1) p += __shfl_xor(p, m, LPC);
    if (!act[k]) continue;
    const size_t bd = row0 + (size_t)k * kCh;
    float* hrow = h + bd * N;
    if (full) {
#pragma unroll
      for (int j = 0; j < SPL; j += 4)
        __builtin_nontemporal_store(f32x4{hv[k][j], hv[k][j + 1], hv[k][j + 2], hv[k][j + 3]},
                                    reinterpret_cast<f32x4*>(hrow + n0 + j));
    } else {
#pragma unroll
      for (int j = 0; j < SPL; ++j)
        if (n0 + j < N) hrow[n0 + j] = hv[k][j];
    }
    if (q == 0) {
      float out = __builtin_fmaf(dd[k], uu[k], p);
      if (z != nullptr) out *= silu(zz[k]);
      if constexpr (BF16) static_cast<uint16_t*>(y)[bd] = f32_to_bf16(out);
      else static_cast<float*>(y)[bd] = out;
    }
  }
}

template <bool BF16, int SPL, int LPC = 4>
hipError_t launch_typed(const UpdateParams& p, hipStream_t stream) {
  constexpr int kCh = 64 / LPC;
  constexpr int kRows = rows_per_thread<LPC>();
  const size_t rows = (size_t)p.batch * p.dim;
  const size_t waves = (rows + kCh * kRows - 1) / (kCh * kRows);
  const unsigned grid = (unsigned)((waves * 64 + kThreadsSU - 1) / kThreadsSU);
  hipLaunchKernelGGL((state_update_kernel<BF16, SPL, LPC>), dim3(grid), dim3(kThreadsSU), 0, stream, p.h, p.u, p.delta,
                     p.A, p.B, p.C, p.D, p.z, p.y, (int)p.batch, (int)p.dim, (int)p.dstate);
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const UpdateParams& p, hipStream_t stream) {
  const int64_t n = p.dstate;
  if (n <= 4) return launch_typed<BF16, 1>(p, stream);
  if (n <= 8) return launch_typed<BF16, 2>(p, stream);
  if (n <= 16) return launch_typed<BF16, 4>(p, stream);
  if (n <= 32) return launch_typed<BF16, 8>(p, stream);
  if (n <= 64) return launch_typed<BF16, 16>(p, stream);
  return launch_typed<BF16, 16, 8>(p, stream);  // up to 128 states: 8 lanes of 16
}

}  // namespace

hipError_t launch_state_update(const UpdateParams& p, hipStream_t stream) {
  return p.bf16 ? launch_dtype<true>(p, stream) : launch_dtype<false>(p, stream);
}

}  // namespace mss
