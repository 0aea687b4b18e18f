// Mamba-3 state update (one generation step) for gfx950.
//
// What is computed (see include/mambascan.h): the Mamba-2 head structure (one
// decay exp(delta*A_h) per head, heads of a group sharing B and C) with the
// three changes "Mamba-1/2/3 visual guide" section 4 gives Mamba-3's
// recurrence: an exponential-trapezoidal input rule (the step's input taken
// at both of its ends), a complex state that rotates while it decays
// (angle delta*theta_n per state), and MIMO (R input vectors and R B/C pairs
// per head: a rank-R update and R outputs).  Per (b, head h, row p, state n):
//   alpha = exp(delta A_h) [* e^{i delta theta[h,n]}]
//   u     = sum_r x[r,p] B[r,n];   u' = sum_r x_prev[r,p] B_prev[r,n]
//   h    <- alpha h + (delta/2)(alpha u' + u)    (trapezoid; else + delta u)
//   y[r,p] = (sum_n C[r,n] Re h[p,n] + D_h x[r,p]) * silu(z[r,p])
//
// Decode streams the state once (read, update, write), so the layout is the
// state update's: a workgroup takes 16 consecutive rows of one head, 16 lanes
// per row, each lane a contiguous slice of SPL states (2*SPL floats when
// complex), so a wave touches 4 whole rows.  Everything a row shares with the
// other rows of its head is formed once per workgroup into LDS: the rotation
// (cos, sin)(delta theta_n) of every state, B, C and B_prev of every rank.
// The R readouts of a row are summed over its 16 lanes in a fixed butterfly
// (bitwise deterministic).  Rank R raises the work per state byte R-fold
// (2R multiply-adds per state for the update and the readout) at the same
// state traffic: the point of MIMO for decode.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace mss {
namespace {

constexpr int kM3Threads = 256;
constexpr int kM3LanesPerRow = 16;
constexpr int kM3Rows = kM3Threads / kM3LanesPerRow;  // rows per workgroup
constexpr int kM3MaxR = 8;
constexpr int kM3MaxN = 256;

template <bool BF16>
__device__ __forceinline__ float ld_io(const void* p, size_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

template <int SPL, bool CPLX, bool TRAP, bool BF16>
__global__ void __launch_bounds__(kM3Threads) mamba3_step_kernel(Mamba3Params a) {
  constexpr int F = CPLX ? 2 * SPL : SPL;  // floats of state per lane
  __shared__ __attribute__((aligned(16))) float s_cs[kM3MaxN][2];  // (cos, sin)(delta theta_n)
  __shared__ __attribute__((aligned(16))) float s_B[kM3MaxR][kM3MaxN];
  __shared__ __attribute__((aligned(16))) float s_C[kM3MaxR][kM3MaxN];
  __shared__ __attribute__((aligned(16))) float s_Bp[TRAP ? kM3MaxR : 1][TRAP ? kM3MaxN : 1];
  __shared__ float s_x[kM3MaxR][kM3Rows], s_xp[TRAP ? kM3MaxR : 1][kM3Rows];

  const int H = (int)a.nheads, P = (int)a.headdim, N = (int)a.dstate, R = (int)a.rank;
  const int hd = blockIdx.y, b = blockIdx.z;
  const int g = hd / (H / (int)a.ngroups);
  const int p0 = blockIdx.x * kM3Rows;
  const int row = threadIdx.x / kM3LanesPerRow, q = threadIdx.x % kM3LanesPerRow;
  const int p = p0 + row;
  const int n0 = q * SPL;
  const size_t bh = (size_t)b * H + hd;
  const size_t bg = (size_t)b * a.ngroups + g;
  const float dl = a.delta[bh];
  const float dec = exp2_fast(dl * a.A[hd] * kLog2e);  // exp(delta A_h)

  // Shared per workgroup: rotations, B, C (and B_prev) of every rank, x (and
  // x_prev) of this workgroup's rows.
  for (int i = threadIdx.x; i < N; i += kM3Threads) {
    if constexpr (CPLX) {
      float sn, cs;
      sincosf(dl * a.theta[(size_t)hd * N + i], &sn, &cs);
      s_cs[i][0] = cs;
      s_cs[i][1] = sn;
    }
  }
  for (int i = threadIdx.x; i < R * N; i += kM3Threads) {
    const int r = i / N, n = i % N;
    const size_t o = (bg * R + r) * N + n;
    s_B[r][n] = ld_io<BF16>(a.B, o);
    s_C[r][n] = ld_io<BF16>(a.C, o);
    if constexpr (TRAP) s_Bp[r][n] = ld_io<BF16>(a.B_prev, o);
  }
  if (threadIdx.x < R * kM3Rows) {
    const int r = threadIdx.x / kM3Rows, rr = threadIdx.x % kM3Rows;
    const size_t o = (bh * R + r) * P + p0 + rr;
    s_x[r][rr] = ld_io<BF16>(a.x, o);
    if constexpr (TRAP) s_xp[r][rr] = ld_io<BF16>(a.x_prev, o);
  }

  // This lane's slice of the state row (whole 16-byte groups: F is a multiple of 4).
  float* hrow = a.h + ((bh * P + p) * N + n0) * (CPLX ? 2 : 1);
  float hv[F];
#pragma unroll
  for (int j = 0; j < F; j += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(hrow + j);
    hv[j] = v[0], hv[j + 1] = v[1], hv[j + 2] = v[2], hv[j + 3] = v[3];
  }
  __syncthreads();

  const float wcur = TRAP ? 0.5f * dl : dl;  // weight of the current input (trapezoid: delta/2)
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    const int n = n0 + j;
    float u = 0.f, up = 0.f;
    for (int r = 0; r < R; ++r) {
      u = __builtin_fmaf(s_x[r][row], s_B[r][n], u);
      if constexpr (TRAP) up = __builtin_fmaf(s_xp[r][row], s_Bp[r][n], up);
    }
    if constexpr (CPLX) {
      const float ar = dec * s_cs[n][0], ai = dec * s_cs[n][1];
      const float re = hv[2 * j], im = hv[2 * j + 1];
      float nre = __builtin_fmaf(ar, re, -ai * im);
      float nim = __builtin_fmaf(ar, im, ai * re);
      if constexpr (TRAP) {
        nre = __builtin_fmaf(wcur, __builtin_fmaf(ar, up, u), nre);
        nim = __builtin_fmaf(wcur * ai, up, nim);
      } else {
        nre = __builtin_fmaf(wcur, u, nre);
      }
      hv[2 * j] = nre;
      hv[2 * j + 1] = nim;
    } else {
      float nh = dec * hv[j];
      if constexpr (TRAP) nh = __builtin_fmaf(wcur, __builtin_fmaf(dec, up, u), nh);
      else nh = __builtin_fmaf(wcur, u, nh);
      hv[j] = nh;
    }
  }
#pragma unroll
  for (int j = 0; j < F; j += 4)
    __builtin_nontemporal_store(f32x4{hv[j], hv[j + 1], hv[j + 2], hv[j + 3]}, reinterpret_cast<f32x4*>(hrow + j));

  // R readouts of the real part, each summed over the row's 16 lanes in a
  // fixed butterfly; lane r of the row finishes output r.
  float mine = 0.f;
  for (int r = 0; r < R; ++r) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < SPL; ++j) acc = __builtin_fmaf(s_C[r][n0 + j], hv[CPLX ? 2 * j : j], acc);
#pragma unroll
    for (int m = 1; m < kM3LanesPerRow; m <<= 1) acc += __shfl_xor(acc, m, kM3LanesPerRow);
    if (q == r) mine = acc;
  }
  if (q < R) {
    const float xv = s_x[q][row];
    float out = __builtin_fmaf(a.D != nullptr ? a.D[hd] : 0.f, xv, mine);
    const size_t o = (bh * R + q) * P + p;
    if (a.z != nullptr) out *= silu(ld_io<BF16>(a.z, o));
    if constexpr (BF16) static_cast<uint16_t*>(a.y)[o] = f32_to_bf16(out);
    else static_cast<float*>(a.y)[o] = out;
  }
}

template <int SPL, bool CPLX, bool TRAP>
hipError_t launch_m3_typed(const Mamba3Params& p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.headdim / kM3Rows), (unsigned)p.nheads, (unsigned)p.batch);
  if (p.bf16) hipLaunchKernelGGL((mamba3_step_kernel<SPL, CPLX, TRAP, true>), grid, dim3(kM3Threads), 0, stream, p);
  else hipLaunchKernelGGL((mamba3_step_kernel<SPL, CPLX, TRAP, false>), grid, dim3(kM3Threads), 0, stream, p);
  return hipGetLastError();
}

template <int SPL>
hipError_t launch_m3_spl(const Mamba3Params& p, hipStream_t stream) {
  const bool cplx = p.theta != nullptr, trap = p.x_prev != nullptr;
  if (cplx) return trap ? launch_m3_typed<SPL, true, true>(p, stream) : launch_m3_typed<SPL, true, false>(p, stream);
  return trap ? launch_m3_typed<SPL, false, true>(p, stream) : launch_m3_typed<SPL, false, false>(p, stream);
}

}  // namespace

hipError_t launch_mamba3_step(const Mamba3Params& p, hipStream_t stream) {
  // dstate is 64, 128 or 256 (validated on the host): 4, 8 or 16 states per
  // lane, whole 16-byte groups of the state row.
  switch (p.dstate / kM3LanesPerRow) {
    case 4: return launch_m3_spl<4>(p, stream);
    case 8: return launch_m3_spl<8>(p, stream);
    default: return launch_m3_spl<16>(p, stream);
  }
}

}  // namespace mss
