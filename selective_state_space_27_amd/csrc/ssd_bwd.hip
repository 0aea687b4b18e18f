// Backward of the Mamba-2 SSD layer on the CDNA4 matrix cores (gfx950).
//
// What is computed (see include/mambascan.h): the gradient of a loss through
// the SSD recurrence ("Mamba-1/2/3 visual guide", section 3: scalar decay per
// head, B and C shared by the heads of a group; the training row of its
// comparison table: the chunked algorithm), given dy = dloss/dy and
// optionally dh_last = dloss/dh_last.  With dyy = dy * silu(z) the gradient
// with respect to the ungated output, G_t the adjoint of the state after
// step t (G_t = dyy_t C_t^T + exp(delta_{t+1} A) G_{t+1}) and h_t the state:
//   dx_t    = delta_t G_t B_t + D dyy_t
//   dB_t    = sum over the group's heads of delta_t G_t^T x_t
//   dC_t    = sum over the group's heads of h_t^T dyy_t
//   ddelta_t = x_t^T G_t B_t + A <G_t, exp(delta_t A) h_{t-1}>
//   dA = sum delta_t <G_t, exp(delta_t A) h_{t-1}>,  dD = sum dyy . x
//   dz = dy * y_ungated * silu'(z),  dh0 = exp(delta_0 A) G_0.
// Blocked the way the page's chunk figures block the forward: 64-step
// blocks, inside a block dense products on the matrix cores, between blocks
// the forward state S and the adjoint E handed along the sequence.  Per block,
// with s_i = A sum_{k<=i} delta_k (prefix sums inside the block), the entering
// state S_in and the adjoint E arriving from the later blocks:
//   G_t = sum_{i>=t} exp(s_i - s_t) dyy_i C_i^T + exp(s_63 - s_t) E
//   h_t = exp(s_t) S_in + sum_{j<=t} exp(s_t - s_j) delta_j x_j B_j^T
// so that, with K = C B^T, W = dyy x^T (64 x 64) and M_ij = exp(s_i - s_j)
// for j <= i (else 0):
//   (G B)^T = E B^T diag(f) + dyy^T (M o K)         f_t = exp(s_63 - s_t)
//   (x^T G)^T = E^T x^T diag(f) + C^T (M o W)
//   (h^T dyy)^T = S_in^T dyy^T diag(e) + B^T (M o W^T o delta)   e_i = exp(s_i)
// and <G_t, exp(delta_t A) h_{t-1}> splits into four sums over the block
// (the i >= t, j < t corner of M o K o W o delta, a suffix sum of
// e_i C_i . (S_in^T dyy_i), a prefix sum of f_j delta_j B_j . (E^T x_j), and
// exp(s_63) <E, S_in>), formed from row and column sums and wave-wide scans.
//
// Passes:
//   1. the forward kernels with 64-step chunks: the state after every block
//      and, with a gate, the ungated output (for dz);
//   2. E along the sequence, from the last block to the first: E_{k-1} =
//      exp(s_63 of block k) E_k + F_k with F_k = sum_i exp(s_i) dyy_i C_i^T
//      (the block's own part of the adjoint handed to the block before), cut
//      into pieces of blocks: each piece's sum from zero, a chain over the
//      pieces, then every block's E from its piece's (dh0 and dz on the way);
//   3. ssd_bwd_grad_kernel: per (block, chunk of a group's virtual heads)
//      every gradient above on the matrix cores; dB and dC as per-chunk
//      parts, ddelta, dA and dD as per-virtual-head parts;
//   4. fixed-order sums of those parts (the results are bitwise repeatable).
// Operands that are not exact bf16 inputs enter the matrix cores as bf16
// hi/lo pairs (two products, three when both operands are split).
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "ssd_common.hpp"

namespace mss {
namespace {

using namespace ssd;

constexpr int kRowP = kP + kPadH;  // row length of the step-major dyy stagings (bf16)

struct BwdArgs {
  const uint16_t* x;      // [b, L, H, P] bf16
  const float* A;         // [H]
  const uint16_t* B;      // [b, L, G, N] bf16
  const uint16_t* C;      // [b, L, G, N] bf16
  const float* D;         // [H] or null
  const uint16_t* z;      // [b, L, H, P] bf16 or null
  const float* h0;        // [b, H, P, N] or null
  const float* dy;        // [b, L, H, P]
  const float* dh_last;   // [b, H, P, N] or null
  float* dx;              // [b, L, H, P]
  float* dz;              // [b, L, H, P], exactly when z is given
  float* ddelta;          // [b, L, H]
  float* dA;              // [H]
  float* dB;              // [b, L, G, N]
  float* dC;              // [b, L, G, N]
  float* dD;              // [H], exactly when D is given
  float* dh0;             // [b, H, P, N] or null
  // Workspace.
  const float* dlT;       // [b, H, Lp]: delta, head-major (0 past L)
  const float* lsT;       // [b, H, Lp]: A log2(e) times the prefix sum of delta inside each 64-step block
  const float* yf;        // [b, L, H, P]: the forward output before the gate
  const float* Sblk;      // [b, nblk, H, P, N]: the state after every block
  float* Eblk;            // [b, nblk, H, P, N]: the adjoint E arriving at every block
  float* Ep;              // [b, npc, H, P, N]: each piece's sum from zero, then the E arriving at its last block
  float* Dp;              // [b, npc, Hv]: each piece's decay (log2)
  float* dBp;             // [b, L, G * cpg, N]: per-chunk parts of dB (hpw virtual heads each)
  float* dCp;             // [b, L, G * cpg, N]: of dC
  float* ddp;             // [b, L, Hv]: of ddelta
  float* dAp;             // [b, nblk, Hv]: of dA
  float* dDp;             // [b, nblk, Hv]: of dD
  int batch, L, H, G, P, ph, Hv, N, nblk, Lp;
  int hpw, cpg, Gc;       // virtual heads per gradient workgroup, chunks per group, G * cpg
  int npc, bpp;           // pieces per sequence for E, blocks per piece
};

// Element offset, inside one step's [H, P] row, of row 0 of virtual head vh
// (rows (vh % ph)*64 .. of head vh / ph).
__device__ __forceinline__ size_t vrow(const BwdArgs& a, int vh) {
  return (size_t)(vh / a.ph) * a.P + (size_t)(vh % a.ph) * kP;
}
// Element offset of virtual head vh's 64 x N state slice in a [lead, H, P, N]
// tensor (rows p at p*N).
__device__ __forceinline__ size_t sbase(const BwdArgs& a, size_t lead, int vh) {
  return (lead * a.H * a.P + vrow(a, vh)) * a.N;
}

__device__ __forceinline__ float sigmoid(float z) { return rcp_fast(1.0f + exp2_fast(-z * kLog2e)); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ f32x4 as_f32x4(u32x4 v) { return __builtin_bit_cast(f32x4, v); }
__device__ __forceinline__ u32x4 as_u32x4(f32x4 v) { return __builtin_bit_cast(u32x4, v); }

// B or C (group g) transposed into a time-contiguous staging T (tsw layout,
// 128 state rows): 512 units of (step pair, 8 states), two per thread; steps
// past L and states past N are staged as zeros.
__device__ __forceinline__ void stage_bc_transposed(const BwdArgs& a, const uint16_t* src, int b, int g, int l0,
                                                    uint16_t* T, int tid) {
  const uint32_t row = (uint32_t)(a.G * a.N * 2);
  const uint32_t left = (uint32_t)max(a.L - l0, 0);
  const rsrc_t r = make_rsrc(src + ((size_t)b * a.L + l0) * a.G * a.N, left * row);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int u = tid + 256 * it;
    const int ng = u & 15, j = 2 * (u >> 4);
    const bool nok = ng * 8 < a.N;
    const uint32_t col = (uint32_t)((g * a.N + ng * 8) * 2);
    const u32x4 r0 = buf_load_u32x4(r, nok ? (uint32_t)j * row + col : kOffNone);
    const u32x4 r1 = buf_load_u32x4(r, nok ? (uint32_t)(j + 1) * row + col : kOffNone);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      *reinterpret_cast<uint32_t*>(&T[tsw(ng * 8 + 2 * k, j)]) = (r0[k] & 0xffffu) | (r1[k] << 16);
      *reinterpret_cast<uint32_t*>(&T[tsw(ng * 8 + 2 * k + 1, j)]) = (r0[k] >> 16) | (r1[k] & 0xffff0000u);
    }
  }
}

// ---------------------------------------------------------------------------
// Pass 2: the adjoint E arriving at every block.  Along the sequence
// E_{k-1} = exp2(ls_63(k)) E_k + F_k, with block k's own part F_k =
// sum_i exp(s_i) dyy_i C_i^T; the blocks are cut into pieces of bpp, and F
// is formed where it is needed (twice) instead of being stored.
//   ssd_bwd_piece_kernel<false>: per (piece, virtual head) the recurrence
//     from zero over the piece's blocks, last to first: its result P into the
//     piece's slot of Ep and the piece's decay (log2) into Dp; dz.
//   ssd_bwd_piece_chain_kernel: along the pieces, last to first, the E
//     arriving at each piece's last block, E_top(j-1) = exp2(Dp_j) E_top(j) +
//     P_j, written over P_j; what arrives before the first block is dh0.
//   ssd_bwd_piece_kernel<true>: per (piece, virtual head) from E_top down
//     the piece, the E arriving at every block into its slot of Eblk.
// grid (npc * Hv, batch), 256 threads.  Wave w forms the states w*32.. (its
// lanes) of F for both 32-row headdim tiles (its registers) and keeps the
// same elements of E: a register of the tile is one row segment of 32
// states, so E is read and written in whole 128-byte lines (waves with
// w*32 >= N only stage).
template <bool WRITE_E>
__global__ void __launch_bounds__(256) ssd_bwd_piece_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t gh[kP * kTRow];  // e o dyy, headdim rows (tsw): hi
  __shared__ __attribute__((aligned(16))) uint16_t gl[kP * kTRow];  // lo
  __shared__ __attribute__((aligned(16))) uint16_t CT[kN * kTRow];  // C, state rows (tsw)
  const int vh = blockIdx.x % a.Hv, pc = blockIdx.x / a.Hv, b = blockIdx.y;
  const int h = vh / a.ph, g = h / (a.H / a.G);
  const int k0 = pc * a.bpp, k1 = min(a.nblk, k0 + a.bpp) - 1;
  // The first piece's sum only feeds dh0: without dh0 (and with no dz to
  // write) the first pass skips it.
  if (!WRITE_E && pc == 0 && !a.dh0 && !a.z) return;
  int lane = threadIdx.x & 63, lc = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const Dot2Masks dm = dot2_masks();
  const int nt = w;
  const bool act = nt * 32 < a.N;
  const float* ls_row = a.lsT + ((size_t)b * a.H + h) * a.Lp;  // + l: s of step l, log2
  float* top = a.Ep + sbase(a, (size_t)b * a.npc + pc, vh);
  // Element (row p, state n) of a 64 x N slice held as register r of tile pt:
  // p = pt*32 + 8(r >> 2) + 4hf + (r & 3), n = nt*32 + lc.
  int n_l = nt * 32 + lc;
  const bool n_ok = n_l < a.N;
  auto tile_off = [&](int pt, int r) { return (size_t)(pt * 32 + 8 * (r >> 2) + 4 * hf + (r & 3)) * a.N + n_l; };
  f32x16 E[2];
#pragma unroll
  for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) E[pt][r] = (WRITE_E && n_ok) ? top[tile_off(pt, r)] : 0.f;
  }
  // A block's loads from memory (dy, and in the first pass z and the ungated
  // y for dz; C; the prefix sums), issued one block ahead of their staging.
  struct Raw {
    u32x4 dy[2][2], z[2], yf[2][2], c[2][2];
    float ls0, ls1, ls63;
  };
  const int pg = threadIdx.x & 7, jx = 2 * (threadIdx.x >> 3);  // dyy: steps jx, jx + 1, rows pg*8 .. +8
  const uint32_t row = (uint32_t)(a.H * a.P), crow = (uint32_t)(a.G * a.N * 2);
  auto issue = [&](int k, Raw& r) {
    const int l0 = k * kSub;
    const uint32_t left = (uint32_t)max(a.L - l0, 0);
    const size_t base = ((size_t)b * a.L + l0) * row + vrow(a, vh);
    const rsrc_t rdy = make_rsrc(a.dy + base, left * row * 4);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const uint32_t o = (uint32_t)(jx + s2) * row + (uint32_t)pg * 8;
      r.dy[s2][0] = buf_load_u32x4(rdy, o * 4);
      r.dy[s2][1] = buf_load_u32x4(rdy, o * 4 + 16);
      if (a.z) {
        const rsrc_t rz = make_rsrc(a.z + base, left * row * 2);
        r.z[s2] = buf_load_u32x4(rz, o * 2);
        if constexpr (!WRITE_E) {
          const rsrc_t ryf = make_rsrc(a.yf + base, left * row * 4);
          r.yf[s2][0] = buf_load_u32x4(ryf, o * 4);
          r.yf[s2][1] = buf_load_u32x4(ryf, o * 4 + 16);
        }
      }
    }
    const rsrc_t rc = make_rsrc(a.C + ((size_t)b * a.L + l0) * a.G * a.N, left * crow);
#pragma unroll
    for (int it = 0; it < 2; ++it) {  // C: (step pair, 8 states) units, two per thread
      const int u = threadIdx.x + 256 * it, ng = u & 15, j = 2 * (u >> 4);
      const uint32_t col = (uint32_t)((g * a.N + ng * 8) * 2);
      r.c[it][0] = buf_load_u32x4(rc, ng * 8 < a.N ? (uint32_t)j * crow + col : kOffNone);
      r.c[it][1] = buf_load_u32x4(rc, ng * 8 < a.N ? (uint32_t)(j + 1) * crow + col : kOffNone);
    }
    r.ls0 = ls_row[l0 + jx];
    r.ls1 = ls_row[l0 + jx + 1];
    r.ls63 = ls_row[l0 + kSub - 1];
  };
  // e o dyy as hi/lo pairs and C transposed into LDS; the first pass writes dz.
  auto stage = [&](const Raw& r, int k) {
    const int l0 = k * kSub;
    const float e[2] = {exp2_fast(r.ls0), exp2_fast(r.ls1)};
    float v[2][8];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const f32x4 d0 = as_f32x4(r.dy[s2][0]), d1 = as_f32x4(r.dy[s2][1]);
      const float dv[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
      if (a.z) {
        float zv[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          zv[2 * q] = bf16_lo(r.z[s2][q]);
          zv[2 * q + 1] = bf16_hi(r.z[s2][q]);
        }
        if constexpr (!WRITE_E) {
          const f32x4 y0 = as_f32x4(r.yf[s2][0]), y1 = as_f32x4(r.yf[s2][1]);
          const float yv[8] = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
          float dzv[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float sg = sigmoid(zv[q]);
            v[s2][q] = dv[q] * (zv[q] * sg);
            dzv[q] = dv[q] * yv[q] * (sg * (1.0f + zv[q] * (1.0f - sg)));
          }
          const uint32_t left = (uint32_t)max(a.L - l0, 0);
          const rsrc_t rdz = make_rsrc(a.dz + ((size_t)b * a.L + l0) * row + vrow(a, vh), left * row * 4);
          const uint32_t o = (uint32_t)(jx + s2) * row + (uint32_t)pg * 8;
          buf_store_u32x4(rdz, o * 4, as_u32x4(f32x4{dzv[0], dzv[1], dzv[2], dzv[3]}));
          buf_store_u32x4(rdz, o * 4 + 16, as_u32x4(f32x4{dzv[4], dzv[5], dzv[6], dzv[7]}));
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) v[s2][q] = dv[q] * silu(zv[q]);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[s2][q] = dv[q];
      }
    }
#pragma unroll
    for (int kq = 0; kq < 8; ++kq) {
      uint32_t hi, lo;
      split2(v[0][kq] * e[0], v[1][kq] * e[1], hi, lo, dm);
      *reinterpret_cast<uint32_t*>(&gh[tsw(pg * 8 + kq, jx)]) = hi;
      *reinterpret_cast<uint32_t*>(&gl[tsw(pg * 8 + kq, jx)]) = lo;
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int u = threadIdx.x + 256 * it, ng = u & 15, j = 2 * (u >> 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w0 = r.c[it][0][q], w1 = r.c[it][1][q];
        *reinterpret_cast<uint32_t*>(&CT[tsw(ng * 8 + 2 * q, j)]) = (w0 & 0xffffu) | (w1 << 16);
        *reinterpret_cast<uint32_t*>(&CT[tsw(ng * 8 + 2 * q + 1, j)]) = (w0 >> 16) | (w1 & 0xffff0000u);
      }
    }
  };

  float dsum = 0.f;  // log2 of the piece's decay
  Raw raw;
  if (!WRITE_E || k1 > k0) issue(k1, raw);
  for (int k = k1; k >= k0; --k) {
    if constexpr (WRITE_E) {
      // Opaque copies of the lane indexes: the 32 store addresses are formed
      // again for every block instead of being held over the loop.
      asm volatile("" : "+v"(hf), "+v"(n_l));
      if (n_ok) {
        float* dst = a.Eblk + sbase(a, (size_t)b * a.nblk + k, vh);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
          for (int r = 0; r < 16; ++r) dst[tile_off(pt, r)] = E[pt][r];
        }
      }
      if (k == k0) break;
    }
    stage(raw, k);
    const float ls63 = raw.ls63;
    dsum += ls63;
    // The next block's loads (the second pass needs none for the piece's
    // first block).
    if (k - 1 >= k0 && !(WRITE_E && k - 1 == k0)) issue(k - 1, raw);
    __syncthreads();
    if (act) {
      f32x16 acc[2] = {};
#pragma unroll
      for (int kk = 0; kk < kSub / 16; ++kk) {
        const int j0 = kk * 16 + 8 * hf;
        const u32x4 cv = *reinterpret_cast<const u32x4*>(&CT[tsw(nt * 32 + lc, j0)]);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          acc[pt] = mfma(*reinterpret_cast<const u32x4*>(&gh[tsw(pt * 32 + lc, j0)]), cv, acc[pt]);
          acc[pt] = mfma(*reinterpret_cast<const u32x4*>(&gl[tsw(pt * 32 + lc, j0)]), cv, acc[pt]);
        }
      }
      const float dq = exp2_fast(ls63);
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) E[pt] = E[pt] * dq + acc[pt];
    }
    __syncthreads();  // the stagings are rewritten for the next block
  }
  if constexpr (!WRITE_E) {
    if (n_ok) {
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) top[tile_off(pt, r)] = E[pt][r];
      }
    }
    if (threadIdx.x == 0) a.Dp[((size_t)b * a.npc + pc) * a.Hv + vh] = dsum;
  }
}

// grid (ceil(16 N / 256) * Hv, batch), 256 threads, 4 state elements per
// thread: from the last piece to the first (the slots hold P_j, loaded four
// pieces ahead; P_0 and its decay, left unwritten without dh0, only reach the
// final E, which is then not stored).
__global__ void __launch_bounds__(256) ssd_bwd_piece_chain_kernel(BwdArgs a) {
  const int xb = (16 * a.N + 255) / 256;
  const int vh = blockIdx.x / xb, b = blockIdx.y;
  const int e = ((blockIdx.x % xb) * 256 + threadIdx.x) * 4;
  if (e >= kP * a.N) return;
  const size_t stride = (size_t)a.H * a.P * a.N;  // from one piece's slot to the next
  float* E0 = a.Ep + sbase(a, (size_t)b * a.npc, vh) + e;
  const float* dp = a.Dp + (size_t)b * a.npc * a.Hv + vh;  // + j*Hv: piece j's decay (log2)
  f32x4 E = a.dh_last ? *reinterpret_cast<const f32x4*>(a.dh_last + sbase(a, b, vh) + e) : f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 P[4];
  float dq[4];
  auto fetch = [&](int j, int s) {
    if (j >= 0) {
      P[s] = *reinterpret_cast<const f32x4*>(E0 + (size_t)j * stride);
      dq[s] = dp[(size_t)j * a.Hv];
    }
  };
  int j = a.npc - 1;
#pragma unroll
  for (int s = 0; s < 4; ++s) fetch(j - s, s);
  for (; j >= 0; j -= 4) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int jj = j - s;
      if (jj < 0) break;
      const f32x4 p = P[s];
      const float d = dq[s];
      fetch(jj - 4, s);
      *reinterpret_cast<f32x4*>(E0 + (size_t)jj * stride) = E;
      E = E * exp2_fast(d) + p;
    }
  }
  if (a.dh0) *reinterpret_cast<f32x4*>(a.dh0 + sbase(a, b, vh) + e) = E;
}

// ---------------------------------------------------------------------------
// Pass 3.  grid (nblk * G * cpg, batch), 512 threads, one workgroup per CU:
// every gradient of one 64-step block for hpw consecutive virtual heads of
// one group (cpg = the group's virtual heads / hpw chunks).  B and C are the
// same for all of them: they are staged once, and K = C B^T (the only product
// that does not involve the head) is formed once and kept in registers; the
// dB and dC parts of the heads are summed in registers, in head order, and
// written once per chunk.  A head's operands (x, dyy, E, S_in) are read from
// memory once, with whole-row loads into registers issued while the head
// before is computed (team 0 loads dyy and x after its first products, team
// 1 E and S_in before its products), and written to LDS (x, dyy as hi/lo in
// two layouts, E and S_in as fp32 rows) between the two heads; the products
// read LDS, and only the step-major B fragments of (G B)^T (L2-resident) and
// the row segments of the outputs touch memory.  Wave 0 assembles each
// head's ddelta and dA, dD parts between the heads.  Two teams of four waves
// run concurrently: team 0 does products 1-3, team 1 products 4.  Wave
// (team, q, sub): q the half of the block whose steps it owns as output
// columns, sub = w & 1.
//   products 1: W(i, j) = dyy_i . x_j for j in half q, i in halves >= q; with
//     K(i, j) = C_i . B_j the column sums of Z = M o K o W o delta (strictly
//     below the diagonal); then M o K and M o W as bf16 hi/lo operands;
//   products 2: (G B)^T for headdim half sub -> dx, x . (G B), dyy . x;
//   products 3: (x^T G)^T for state tiles 2 sub, 2 sub + 1 -> dB part and
//     B . (E^T x);
//   products 4: W^T(j, i) for i in half q, j in halves <= q, with K^T the row
//     sums of Z, then (h^T dyy)^T for the same state tiles -> dC part and
//     C . (S_in^T dyy);
//   then wave 0 (lane = step) assembles ddelta and the dA and dD parts.
constexpr int kERow = kN + 4;  // row length (floats) of the E staging

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads() it
// does not first wait for this wave's direct-to-LDS loads (whose data only
// the wave that issued them reads, after waiting for them itself).
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Position of S_in element (row p, state n) in its staging: the two 64-state
// halves one after the other, each as 64 rows of 64 states in 4-state groups;
// in rows p with bit 3 set, bit 3 of the group index is flipped, so that a
// column read of rows p and p + 8 by one wave touches every bank once.  A
// direct-to-LDS load writes 64 consecutive groups (4 rows): the swizzle is
// applied to the addresses it reads.
__device__ __forceinline__ int ss_index(int p, int n) {
  return (n >> 6) * (kP * 64) + p * 64 + (((((n & 63) >> 2) ^ (((p >> 3) & 1) << 3))) << 2) + (n & 3);
}

__global__ void __launch_bounds__(512, 1) ssd_bwd_grad_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t dyRh[kSub][kRowP];  // dyy, step rows: hi
  __shared__ __attribute__((aligned(16))) uint16_t dyRl[kSub][kRowP];  // lo
  __shared__ __attribute__((aligned(16))) uint16_t BT[kN * kTRow];     // B, state rows (tsw)
  __shared__ __attribute__((aligned(16))) uint16_t CT[kN * kTRow];     // C, state rows (tsw)
  __shared__ __attribute__((aligned(16))) uint16_t xs[kSub][kRowP];    // x, step rows
  __shared__ __attribute__((aligned(16))) uint16_t Bq0[32][kN + kPadH];  // B, steps 0..31 (0 past N)
  __shared__ __attribute__((aligned(16))) float Es[kP * kERow];        // E [p][n] (0 past N)
  __shared__ __attribute__((aligned(16))) float Ss[kP * kN];           // S_in (layout: ss_index; 0 past N)
  // Step values of the block (delta, s, exp(s), exp(s_63 - s)), double-buffered
  // over the heads: the next head's are written while this head's assembly
  // still reads them.
  __shared__ __attribute__((aligned(16))) float s_dl[2][kSub], s_ls[2][kSub], s_e[2][kSub], s_f[2][kSub];
  __shared__ float s_col[kSub], s_row[kSub], s_T[2][kSub], s_U[2][kSub], s_c[2][kSub];
  __shared__ float s_es[4], s_dd[4];

  const int gc = blockIdx.x % a.Gc, blk = blockIdx.x / a.Gc, b = blockIdx.y;
  const int g = gc / a.cpg;
  const int vh0 = g * (a.Hv / a.G) + (gc % a.cpg) * a.hpw;  // the chunk's first virtual head
  const int l0 = blk * kSub;
  // Lane indexes (re-derived opaquely for every head: see the head loop).
  int lane = threadIdx.x & 63, lc = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int team = w >> 2, q = (w >> 1) & 1, sub = w & 1;
  const Dot2Masks dm = dot2_masks();
  const int nk = a.N / 16;  // 16-state k-steps
  const uint32_t left = (uint32_t)max(a.L - l0, 0);
  const uint32_t xrow = (uint32_t)(a.H * a.P), brow = (uint32_t)(a.G * a.N);
  const size_t bbase = ((size_t)b * a.L + l0) * brow + (size_t)g * a.N;
  const rsrc_t rb = make_rsrc(a.B + bbase, left * brow * 2);
  const rsrc_t rc = make_rsrc(a.C + bbase, left * brow * 2);
  // Every k loop runs over all 128 states (8 steps of 16) so that it unrolls;
  // states past N read 0.
  constexpr int kNK = kN / 16;
  // B or C rows of step T*32 + lc, states kk*16 + 8hf .. +8 (A rows or B columns).
  auto frag_bc = [&](rsrc_t r, int T, int kk) -> u32x4 {
    return buf_load_u32x4(r, kk < nk ? ((uint32_t)(T * 32 + lc) * brow + (uint32_t)(kk * 16 + 8 * hf)) * 2
                                     : kOffNone);
  };
  auto xbase = [&](int vh) { return ((size_t)b * a.L + l0) * xrow + vrow(a, vh); };
  // The state entering the block (S_in) of virtual head vh, or null.
  auto sin_ptr = [&](int vh) -> const float* {
    return blk > 0 ? a.Sblk + sbase(a, (size_t)b * a.nblk + blk - 1, vh) : (a.h0 ? a.h0 + sbase(a, b, vh) : nullptr);
  };

  // ---- the per-head stagings, in two halves: loads into registers and their
  // writes to LDS.  Of the first head, team 0 moves dyy and x, team 1 E, S_in
  // and (wave 4) the step values delta and s; of every later head, team 1
  // moves all of them: it issues the loads as it starts the head before (its
  // registers allow it) and writes LDS after the barrier that ends that head.
  struct T0Regs {
    u32x4 dy[2][2], z[2], x[2];
  };
  struct T1Regs {
    u32x4 e[kP * kN / 4 / 256];
    float dl, ls;
  };
  // The staging addresses are formed from an opaque copy of the thread index
  // (taken mod 256: the thread's index in its team)
  // so that they are formed again for every head instead of being held (in
  // registers that the products need) over the head loop.
  auto opaque_tid = [] {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
  };
  auto issue_t0 = [&](int vh, T0Regs& r) {
    const int t = opaque_tid() & 255, pg = t & 7, jx = 2 * (t >> 3);
    const size_t xb = xbase(vh);
    const rsrc_t rdy = make_rsrc(a.dy + xb, left * xrow * 4);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t o = (uint32_t)(jx + s) * xrow + (uint32_t)pg * 8;  // dyy: steps jx, jx + 1, rows pg*8 .. +8
      r.dy[s][0] = buf_load_u32x4(rdy, o * 4);
      r.dy[s][1] = buf_load_u32x4(rdy, o * 4 + 16);
    }
    if (a.z) {
      const rsrc_t rz = make_rsrc(a.z + xb, left * xrow * 2);
#pragma unroll
      for (int s = 0; s < 2; ++s) r.z[s] = buf_load_u32x4(rz, ((uint32_t)(jx + s) * xrow + (uint32_t)pg * 8) * 2);
    }
    const rsrc_t rx = make_rsrc(a.x + xb, left * xrow * 2);
#pragma unroll
    for (int k = 0; k < 2; ++k) {  // x: step u / 8, headdim rows (u % 8) * 8 .. +8
      const int u = t + 256 * k, st = u >> 3, pc = (u & 7) * 8;
      r.x[k] = buf_load_u32x4(rx, ((uint32_t)st * xrow + (uint32_t)pc) * 2);
    }
  };
  auto commit_t0 = [&](const T0Regs& r) {
    const int t = opaque_tid() & 255, pg = t & 7, jx = 2 * (t >> 3);
    float v[2][8];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f32x4 d0 = as_f32x4(r.dy[s][0]), d1 = as_f32x4(r.dy[s][1]);
      const float dv[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
#pragma unroll
      for (int k = 0; k < 8; ++k) v[s][k] = dv[k];
      if (a.z) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[s][2 * k] *= silu(bf16_lo(r.z[s][k]));
          v[s][2 * k + 1] *= silu(bf16_hi(r.z[s][k]));
        }
      }
      u32x4 hi, lo;
      split8(v[s], hi, lo, dm);
      *reinterpret_cast<u32x4*>(&dyRh[jx + s][pg * 8]) = hi;
      *reinterpret_cast<u32x4*>(&dyRl[jx + s][pg * 8]) = lo;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int u = t + 256 * k, st = u >> 3, pc = (u & 7) * 8;
      *reinterpret_cast<u32x4*>(&xs[st][pc]) = r.x[k];
    }
  };
  // The fewest loads from memory a team-1 wave issues for the next head's
  // operands (E 8, dyy 4, x 2; z and the step values add to them).
  constexpr int kOperandLoadsMin = kP * kN / 4 / 256 + 4 + 2;
  // E: whole 16-byte groups of its 64 x N slice; states past N read 0.
  auto issue_t1 = [&](int vh, T1Regs& r) {
    const int t = opaque_tid() & 255;
    if (w == 4) {
      const size_t o = ((size_t)b * a.H + vh / a.ph) * a.Lp + l0 + lane;
      r.dl = a.dlT[o];
      r.ls = a.lsT[o];
    }
    const rsrc_t rE = make_rsrc(a.Eblk + sbase(a, (size_t)b * a.nblk + blk, vh), (uint32_t)(kP * a.N * 4));
#pragma unroll
    for (int it = 0; it < kP * kN / 4 / 256; ++it) {
      const int e4 = t + 256 * it, pr = e4 >> 5, n = (e4 & 31) * 4;
      r.e[it] = buf_load_u32x4(rE, n < a.N ? ((uint32_t)pr * a.N + (uint32_t)n) * 4 : kOffNone);
    }
  };
  // S_in straight from memory into its staging (direct-to-LDS loads: no
  // registers), by team 1, whose products alone read it: wave (q, sub) loads
  // the half of the states it reads, 16 loads of 4 rows each (the two waves of
  // a half write the same values).  States past N and an absent S_in are
  // written as 0.  A wave's reads of the staging wait for its own loads.
  auto dma_s = [&](int vh) {
    const int t = opaque_tid() & 63;
    const float* Sp = sin_ptr(vh);
    const rsrc_t rS = make_rsrc(Sp, Sp ? (uint32_t)(kP * a.N * 4) : 0u);
    const int pl = t >> 4, gs = t & 15;  // row in the load's 4, swizzled group
#pragma unroll
    for (int j = 0; j < kP / 4; ++j) {
      const int p = 4 * j + pl, n = sub * 64 + ((gs ^ (((p >> 3) & 1) << 3)) << 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rS, (__attribute__((address_space(3))) void*)(Ss + sub * (kP * 64) + j * 256), 16,
          n < a.N ? ((uint32_t)p * a.N + (uint32_t)n) * 4 : kOffNone, 0, 0, 0);
    }
  };
  auto commit_t1 = [&](const T1Regs& r, int pw) {
    const int t = opaque_tid() & 255;
    if (w == 4) {
      const float ls63 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r.ls), 63));
      s_dl[pw][lane] = r.dl;
      s_ls[pw][lane] = r.ls;
      s_e[pw][lane] = exp2_fast(r.ls);
      s_f[pw][lane] = exp2_fast(ls63 - r.ls);
    }
#pragma unroll
    for (int it = 0; it < kP * kN / 4 / 256; ++it) {
      const int e4 = t + 256 * it, pr = e4 >> 5, n = (e4 & 31) * 4;
      *reinterpret_cast<u32x4*>(&Es[pr * kERow + n]) = r.e[it];
    }
  };

  // The first head's stagings and B, C (time-contiguous), with K (team 0:
  // K = C B^T, columns in half q, row halves q + u) or K^T (team 1: K^T =
  // B C^T, columns in half q, row halves u <= q) formed from step-major B and
  // C fragments read from memory (L2-resident: the group's other chunks read
  // them too) and issued first, so that their latency hides behind the
  // stagings.
  f32x16 kk2[2] = {};
  {
    u32x4 f1[kNK], f2[2][kNK];
    const rsrc_t r1 = team == 0 ? rb : rc, r2 = team == 0 ? rc : rb;
#pragma unroll
    for (int kk = 0; kk < kNK; ++kk) f1[kk] = frag_bc(r1, q, kk);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bool use = team == 0 ? q + u <= 1 : u <= q;
      const int rows = team == 0 ? q + u : u;
#pragma unroll
      for (int kk = 0; kk < kNK; ++kk) f2[u][kk] = use ? frag_bc(r2, rows, kk) : u32x4{0u, 0u, 0u, 0u};
    }
    if (team == 0) {
      T0Regs r;
      issue_t0(vh0, r);
      stage_bc_transposed(a, a.C, b, g, l0, CT, threadIdx.x);
#pragma unroll
      for (int it = 0; it < 2; ++it) {  // B rows of the first half, step-major
        const int u = threadIdx.x + 256 * it, row = u >> 4, n = (u & 15) * 8;
        *reinterpret_cast<u32x4*>(&Bq0[row][n]) =
            buf_load_u32x4(rb, n < a.N ? ((uint32_t)row * brow + (uint32_t)n) * 2 : kOffNone);
      }
      commit_t0(r);
    } else {
      T1Regs r;
      dma_s(vh0);
      issue_t1(vh0, r);
      stage_bc_transposed(a, a.B, b, g, l0, BT, threadIdx.x - 256);
      commit_t1(r, 0);
    }
#pragma unroll
    for (int kk = 0; kk < kNK; ++kk) {
#pragma unroll
      for (int u = 0; u < 2; ++u) kk2[u] = mfma(f2[u][kk], f1[kk], kk2[u]);
    }
  }
  __syncthreads();

  // ---- operand fragments
  // x of step T*32 + lc, headdim rows kp*16 + 8hf .. +8.
  auto frag_x = [&](int T, int kp) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(&xs[T * 32 + lc][kp * 16 + 8 * hf]);
  };
  // dyy (hi or lo) as the headdim-row operand: row p = sub*32 + lc, steps
  // i0 .. i0 + 7 (i0 includes 8hf), read from the step-major staging with two
  // transposing LDS reads.  ds_read_b64_tr_b16 gives lane i of each 16-lane
  // group, as value q, 16-bit element i % 4 of the 8 bytes addressed by lane
  // 4q + i / 4 of the group; so lane i addresses steps i0 + i / 4 (+ 4),
  // headdim rows sub*32 + 16 (group & 1) + 4 (i % 4) .. +4.
  auto frag_tr = [&](const uint16_t (*R)[kRowP], int i0) -> u32x4 {
    typedef short v4s __attribute__((ext_vector_type(4)));
    const int i = lane & 15;
    const uint16_t* p0 = &R[i0 + (i >> 2)][sub * 32 + 16 * ((lane >> 4) & 1) + 4 * (i & 3)];
    const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p0));
    const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p0 + 4 * kRowP));
    const u32x2 a2 = __builtin_bit_cast(u32x2, lo4), b2 = __builtin_bit_cast(u32x2, hi4);
    return u32x4{a2[0], a2[1], b2[0], b2[1]};
  };
  // E staging: rows p = PT*32 + lc, states kk*16 + 8hf .. +8.
  auto ld_srow = [&](const float* S, int PT, int kk, float* v) {
    const float* r = S + (PT * 32 + lc) * kERow + kk * 16 + 8 * hf;
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(r), v1 = *reinterpret_cast<const f32x4*>(r + 4);
    v[0] = v0[0], v[1] = v0[1], v[2] = v0[2], v[3] = v0[3], v[4] = v1[0], v[5] = v1[1], v[6] = v1[2], v[7] = v1[3];
  };
  // E staging: state n = NT*32 + lc, rows kp*16 + 8hf + t.
  auto ld_scol = [&](const float* S, int NT, int kp, float* v) {
    const float* r = S + (kp * 16 + 8 * hf) * kERow + NT * 32 + lc;
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = r[t * kERow];
  };
  // S_in staging: state n = NT*32 + lc, rows kp*16 + 8hf + t.
  auto ld_scol_s = [&](int NT, int kp, float* v) {
    const float* r = Ss + ss_index(kp * 16 + 8 * hf, NT * 32 + lc);
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = r[t * 64];
  };
  auto lds4 = [](const float* p) { return *reinterpret_cast<const f32x4*>(p); };

  int col = q * 32 + lc;  // this lane's output column: step (of the block) of every tile below
  // The chunk's dB (team 0) or dC (team 1) part for state tiles 2 sub + v, column col.
  f32x16 dacc[2] = {};

  int par = 0;  // the current head's buffer of the step values
  auto body = [&](auto qtag, auto team_tag, int vh, bool next, T0Regs& p0, T1Regs& p1, const u32x4* fb1) {
    constexpr int Q = decltype(qtag)::value;
    constexpr int NI = 2 - Q;  // row halves Q..1 (products 1)
    constexpr int NJ = Q + 1;  // row halves 0..Q (products 4)
    constexpr int TEAM = decltype(team_tag)::value;
    const float ls_c = s_ls[par][col], dl_c = s_dl[par][col];

    if constexpr (TEAM == 0) {
    // ---- products 1: W, rows i in halves >= Q, columns j = col
    u32x4 mkh[NI][2], mkl[NI][2], mwh[NI][2], mwl[NI][2];
    {
      f32x16 wacc[NI] = {};
#pragma unroll
      for (int kp = 0; kp < kP / 16; ++kp) {
        const u32x4 xop = frag_x(Q, kp);
#pragma unroll
        for (int u = 0; u < NI; ++u) {
          wacc[u] = mfma(*reinterpret_cast<const u32x4*>(&dyRh[(Q + u) * 32 + lc][kp * 16 + 8 * hf]), xop, wacc[u]);
          wacc[u] = mfma(*reinterpret_cast<const u32x4*>(&dyRl[(Q + u) * 32 + lc][kp * 16 + 8 * hf]), xop, wacc[u]);
        }
      }
      // M o K and M o W (i >= j) in the accumulator layout (each M_ij formed
      // once), the column sums of Z below the diagonal (i > j) from them, then
      // both as operands: k = i, column j.
      float cs = 0.f;
#pragma unroll
      for (int u = 0; u < NI; ++u) {
        f32x16 mk;
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const int i0 = (Q + u) * 32 + 8 * k4 + 4 * hf;
          const f32x4 lsi = lds4(&s_ls[par][i0]);
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const int r = 4 * k4 + qq;
            const float m = (i0 + qq >= col) ? exp2_fast(lsi[qq] - ls_c) : 0.f;
            mk[r] = m * kk2[u][r];
            cs += (i0 + qq > col ? mk[r] : 0.f) * wacc[u][r];
            wacc[u][r] *= m;
          }
        }
        auto slice = [&](auto stag) {
          constexpr int S = decltype(stag)::value;
          float kv[8], wv[8];
          acc_kslice<S>(mk, kv);
          acc_kslice<S>(wacc[u], wv);
          split8(kv, mkh[u][S], mkl[u][S], dm);
          split8(wv, mwh[u][S], mwl[u][S], dm);
        };
        slice(std::integral_constant<int, 0>{});
        slice(std::integral_constant<int, 1>{});
      }
      cs = (cs + __shfl_xor(cs, 32)) * dl_c;
      if (sub == 0 && hf == 0) s_col[col] = cs;
    }

    // ---- products 2: (G B)^T, headdim rows sub*32.., columns col
    {
      f32x16 gacc = {};
#pragma unroll
      for (int kk = 0; kk < kNK; ++kk) {
        float ev[8];
        ld_srow(Es, sub, kk, ev);
        u32x4 eh, el;
        split8(ev, eh, el, dm);
        const u32x4 bop = Q == 1 ? fb1[kk] : *reinterpret_cast<const u32x4*>(&Bq0[lc][kk * 16 + 8 * hf]);
        gacc = mfma(eh, bop, gacc);
        gacc = mfma(el, bop, gacc);
      }
      gacc *= s_f[par][col];
#pragma unroll
      for (int u = 0; u < NI; ++u) {
#pragma unroll
        for (int S = 0; S < 2; ++S) {
          const int i0 = (Q + u) * 32 + 16 * S + 8 * hf;
          const u32x4 ah = frag_tr(dyRh, i0), al = frag_tr(dyRl, i0);
          gacc = mfma(ah, mkh[u][S], gacc);
          gacc = mfma(al, mkh[u][S], gacc);
          gacc = mfma(ah, mkl[u][S], gacc);
        }
      }
      // dx, x . (G B) and dyy . x for (step col, rows p); dyy as its staged
      // hi + lo pair (within 2^-17 of the fp32 value).
      const rsrc_t rdx = make_rsrc(a.dx + xbase(vh), left * xrow * 4);
      const float Dh = a.D ? a.D[vh / a.ph] : 0.f;
      float cp = 0.f, dd = 0.f;
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int p0 = sub * 32 + 8 * k4 + 4 * hf;
        const uint32_t o = (uint32_t)col * xrow + (uint32_t)p0;
        const u32x2 xx = *reinterpret_cast<const u32x2*>(&xs[col][p0]);
        const u32x2 yh = *reinterpret_cast<const u32x2*>(&dyRh[col][p0]);
        const u32x2 yl = *reinterpret_cast<const u32x2*>(&dyRl[col][p0]);
        const float xv[4] = {bf16_lo(xx[0]), bf16_hi(xx[0]), bf16_lo(xx[1]), bf16_hi(xx[1])};
        const float yv[4] = {bf16_lo(yh[0]) + bf16_lo(yl[0]), bf16_hi(yh[0]) + bf16_hi(yl[0]),
                             bf16_lo(yh[1]) + bf16_lo(yl[1]), bf16_hi(yh[1]) + bf16_hi(yl[1])};
        f32x4 dxv;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const float gb = gacc[4 * k4 + qq], dyy = yv[qq];
          cp += xv[qq] * gb;
          dd += dyy * xv[qq];
          dxv[qq] = dl_c * gb + Dh * dyy;
        }
        buf_store_u32x4(rdx, o * 4, as_u32x4(dxv));
      }
      cp += __shfl_xor(cp, 32);
      if (hf == 0) s_c[sub][col] = cp;
      dd = wave_sum(dd);
      if (lane == 0) s_dd[w] = dd;
    }

    // ---- products 3: (x^T G)^T, state tiles 2 sub + v, columns col
    {
      float up = 0.f;
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int NT = 2 * sub + v;
        if (NT * 32 >= a.N) continue;
        f32x16 xacc = {};
#pragma unroll
        for (int kp = 0; kp < kP / 16; ++kp) {
          float ev[8];
          ld_scol(Es, NT, kp, ev);
          u32x4 eh, el;
          split8(ev, eh, el, dm);
          const u32x4 xop = frag_x(Q, kp);
          xacc = mfma(eh, xop, xacc);
          xacc = mfma(el, xop, xacc);
        }
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          const int n0 = NT * 32 + 8 * k4 + 4 * hf;
          // B of step col, states n0 .. n0 + 3 (the staged rows past N are 0)
          up += xacc[4 * k4] * bf16_to_f32(BT[tsw(n0, col)]) + xacc[4 * k4 + 1] * bf16_to_f32(BT[tsw(n0 + 1, col)]) +
                xacc[4 * k4 + 2] * bf16_to_f32(BT[tsw(n0 + 2, col)]) +
                xacc[4 * k4 + 3] * bf16_to_f32(BT[tsw(n0 + 3, col)]);
        }
        xacc *= s_f[par][col];
#pragma unroll
        for (int u = 0; u < NI; ++u) {
#pragma unroll
          for (int S = 0; S < 2; ++S) {
            const int i0 = (Q + u) * 32 + 16 * S + 8 * hf;
            const u32x4 av = *reinterpret_cast<const u32x4*>(&CT[tsw(NT * 32 + lc, i0)]);
            xacc = mfma(av, mwh[u][S], xacc);
            xacc = mfma(av, mwl[u][S], xacc);
          }
        }
        dacc[v] += dl_c * xacc;
      }
      up += __shfl_xor(up, 32);
      if (hf == 0) s_U[sub][col] = up;
    }

    }  // team 0
    if constexpr (TEAM == 1) {
    // The next head's operands, in flight until the stagings (the products
    // below read only LDS: a load's result would wait for every load issued
    // before it).
    if (next) {
      issue_t1(vh + 1, p1);
      issue_t0(vh + 1, p0);
    }
    // ---- products 4: W^T (rows j in halves <= Q, columns i = col), with K^T
    // the row sums of Z, then (h^T dyy)^T for state tiles 2 sub + v.
    {
      u32x4 mth[NJ][2], mtl[NJ][2];
      {
        f32x16 wt[NJ] = {};
#pragma unroll
        for (int kp = 0; kp < kP / 16; ++kp) {
          const u32x4 dh = *reinterpret_cast<const u32x4*>(&dyRh[col][kp * 16 + 8 * hf]);
          const u32x4 dl = *reinterpret_cast<const u32x4*>(&dyRl[col][kp * 16 + 8 * hf]);
#pragma unroll
          for (int u = 0; u < NJ; ++u) {
            const u32x4 xa = frag_x(u, kp);
            wt[u] = mfma(xa, dh, wt[u]);
            wt[u] = mfma(xa, dl, wt[u]);
          }
        }
        // M o W^T o delta_j (j <= i) in the accumulator layout (each weight
        // formed once), the row sums of Z left of the diagonal (j < i) from it,
        // then as operands: k = j, column i.
        float rs = 0.f;
#pragma unroll
        for (int u = 0; u < NJ; ++u) {
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4) {
            const int j0 = u * 32 + 8 * k4 + 4 * hf;
            const f32x4 lsj = lds4(&s_ls[par][j0]), dlj = lds4(&s_dl[par][j0]);
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              const int r = 4 * k4 + qq;
              const float m = (j0 + qq <= col) ? exp2_fast(ls_c - lsj[qq]) * dlj[qq] : 0.f;
              wt[u][r] = m * wt[u][r];
              rs += (j0 + qq < col ? wt[u][r] : 0.f) * kk2[u][r];
            }
          }
        }
        rs += __shfl_xor(rs, 32);
        if (sub == 0 && hf == 0) s_row[col] = rs;
#pragma unroll
        for (int u = 0; u < NJ; ++u) {
          auto slice = [&](auto stag) {
            constexpr int S = decltype(stag)::value;
            float v[8];
            acc_kslice<S>(wt[u], v);
            split8(v, mth[u][S], mtl[u][S], dm);
          };
          slice(std::integral_constant<int, 0>{});
          slice(std::integral_constant<int, 1>{});
        }
      }
      const bool has_sin = sin_ptr(vh) != nullptr;
      // This wave's direct-to-LDS loads of S_in (issued before this head
      // began) must have landed; the compiler does not track them over the
      // head loop.  Only the next head's operand loads, issued after them, may
      // still be in flight.
      if (next)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kOperandLoadsMin) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      float tp = 0.f, es = 0.f;
      const float ec = s_e[par][col];
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int NT = 2 * sub + v;
        if (NT * 32 >= a.N) continue;
        f32x16 cacc = {};
        if (has_sin) {
#pragma unroll
          for (int kp = 0; kp < kP / 16; ++kp) {
            float sv[8];
            ld_scol_s(NT, kp, sv);
            if (Q == 0) {  // <E, S_in>: each element once, over the two Q = 0 waves
              float ev[8];
              ld_scol(Es, NT, kp, ev);
#pragma unroll
              for (int t = 0; t < 8; ++t) es += ev[t] * sv[t];
            }
            u32x4 sh, sl;
            split8(sv, sh, sl, dm);
            const u32x4 bh = *reinterpret_cast<const u32x4*>(&dyRh[col][kp * 16 + 8 * hf]);
            const u32x4 bl = *reinterpret_cast<const u32x4*>(&dyRl[col][kp * 16 + 8 * hf]);
            cacc = mfma(sh, bh, cacc);
            cacc = mfma(sh, bl, cacc);
            cacc = mfma(sl, bh, cacc);
          }
#pragma unroll
          for (int k4 = 0; k4 < 4; ++k4) {
            const int n0 = NT * 32 + 8 * k4 + 4 * hf;
            // C of step col, states n0 .. n0 + 3 (the staged rows past N are 0)
            tp += cacc[4 * k4] * bf16_to_f32(CT[tsw(n0, col)]) + cacc[4 * k4 + 1] * bf16_to_f32(CT[tsw(n0 + 1, col)]) +
                  cacc[4 * k4 + 2] * bf16_to_f32(CT[tsw(n0 + 2, col)]) +
                  cacc[4 * k4 + 3] * bf16_to_f32(CT[tsw(n0 + 3, col)]);
          }
          cacc *= ec;
        }
#pragma unroll
        for (int u = 0; u < NJ; ++u) {
#pragma unroll
          for (int S = 0; S < 2; ++S) {
            const int j0 = u * 32 + 16 * S + 8 * hf;
            const u32x4 av = *reinterpret_cast<const u32x4*>(&BT[tsw(NT * 32 + lc, j0)]);
            cacc = mfma(av, mth[u][S], cacc);
            cacc = mfma(av, mtl[u][S], cacc);
          }
        }
        dacc[v] += cacc;
      }
      tp += __shfl_xor(tp, 32);
      if (hf == 0) s_T[sub][col] = tp;
      es = wave_sum(es);
      if (lane == 0) s_es[w & 3] = es;
    }
    }
  };

  // The head loop, inside each wave kind's own copy of the code (its values
  // that do not change over the heads then stay its own).
  auto run = [&](auto qtag, auto team_tag) {
    constexpr int TEAM = decltype(team_tag)::value;
    constexpr int Q = decltype(qtag)::value;
    T0Regs p0;
    T1Regs p1;
    // The B fragments of (G B)^T: the half-1 waves of team 0 (registers to
    // spare) keep theirs over the heads, the half-0 waves read theirs from
    // the step-major staging of the first half.
    u32x4 fb1[TEAM == 0 && Q == 1 ? kNK : 1];
    if constexpr (TEAM == 0 && Q == 1) {
#pragma unroll
      for (int kk = 0; kk < kNK; ++kk) fb1[kk] = frag_bc(rb, 1, kk);
    }
    for (int i = 0; i < a.hpw; ++i) {
      const int vh = vh0 + i;
      const bool next = i + 1 < a.hpw;
      // Opaque copies of the lane indexes: the addresses formed from them are
      // then formed again for every head instead of being held over the loop.
      asm volatile("" : "+v"(lane), "+v"(lc), "+v"(hf));
      col = q * 32 + lc;
      par = i & 1;
      body(qtag, team_tag, vh, next, p0, p1, fb1);
      __syncthreads();

      // ---- ddelta and the dA, dD parts (lane = step of the block), by wave 0
      // while team 1 writes the next head's stagings (no LDS that this reads:
      // the step values are double-buffered).
      if (w == 0) {
        const int t = lane;
        const float dl = s_dl[par][t], e = s_e[par][t], f = s_f[par][t];
        const float cprime = s_c[0][t] + s_c[1][t];
        const float cr = s_col[t] - s_row[t];
        const float corner = wave_prefix_sum(cr) - cr;  // R_t: sum over u < t
        const float et = e * (s_T[0][t] + s_T[1][t]);
        const float pt = wave_prefix_sum(et);
        const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pt), 63));
        const float suffix = tot - (pt - et);  // sum over i >= t
        const float fu = f * dl * (s_U[0][t] + s_U[1][t]);
        const float prefix = wave_prefix_sum(fu) - fu;  // sum over j < t
        const float dq63 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e), 63));
        const float es = (s_es[0] + s_es[1]) + (s_es[2] + s_es[3]);
        const float gh = corner + suffix + prefix + dq63 * es;  // <G_t, exp(delta_t A) h_{t-1}>
        if (l0 + t < a.L) a.ddp[((size_t)b * a.L + l0 + t) * a.Hv + vh] = cprime + a.A[vh / a.ph] * gh;
        const float da = wave_sum(dl * gh);
        if (lane == 0) {
          const size_t o = ((size_t)b * a.nblk + blk) * a.Hv + vh;
          a.dAp[o] = da;
          a.dDp[o] = (s_dd[0] + s_dd[1]) + (s_dd[2] + s_dd[3]);
        }
      }
      if (next) {
        if constexpr (TEAM == 1) {
          commit_t1(p1, par ^ 1);
          commit_t0(p0);
          // After the writes above: a write to LDS waits for the direct-to-LDS
          // loads issued before it.
          dma_s(vh + 1);
        }
        barrier_lds();
      }
    }
  };
  if (team == 0) {
    if (q == 0) run(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
  } else {
    if (q == 0) run(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
    else run(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
  }

  // ---- the chunk's dB (team 0) and dC (team 1) parts, row (b, l0 + col, g, chunk)
  if (l0 + col < a.L) {
    float* dst = (team == 0 ? a.dBp : a.dCp) + (((size_t)b * a.L + l0 + col) * a.Gc + gc) * a.N;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int n0 = (2 * sub + v) * 32 + 8 * k4 + 4 * hf;
        if (n0 < a.N)
          *reinterpret_cast<f32x4*>(dst + n0) =
              f32x4{dacc[v][4 * k4], dacc[v][4 * k4 + 1], dacc[v][4 * k4 + 2], dacc[v][4 * k4 + 3]};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Pass 4: fixed-order sums of the parts.
// dB and dC: grid-stride over (b, l, g, 4 states), the group's chunks summed
// in order.
__global__ void __launch_bounds__(256) ssd_bwd_reduce_bc_kernel(BwdArgs a) {
  const int n4s = a.N / 4;
  const size_t total = (size_t)a.batch * a.L * a.G * n4s;
  for (size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (size_t)gridDim.x * 256) {
    const int n4 = (int)(idx % n4s);
    const size_t rest = idx / n4s;
    const int g = (int)(rest % a.G);
    const size_t bl = rest / a.G;  // b*L + l
    const size_t src = (bl * a.Gc + (size_t)g * a.cpg) * a.N + 4 * n4;
    f32x4 sb = {0.f, 0.f, 0.f, 0.f}, sc = {0.f, 0.f, 0.f, 0.f};
    for (int v = 0; v < a.cpg; ++v) {
      sb += *reinterpret_cast<const f32x4*>(a.dBp + src + (size_t)v * a.N);
      sc += *reinterpret_cast<const f32x4*>(a.dCp + src + (size_t)v * a.N);
    }
    const size_t dst = (bl * a.G + g) * a.N + 4 * n4;
    *reinterpret_cast<f32x4*>(a.dB + dst) = sb;
    *reinterpret_cast<f32x4*>(a.dC + dst) = sc;
  }
}

// ddelta: grid-stride over (b, l, h), the head's ph virtual heads in order.
__global__ void __launch_bounds__(256) ssd_bwd_reduce_dd_kernel(BwdArgs a) {
  const size_t total = (size_t)a.batch * a.L * a.H;
  for (size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (size_t)gridDim.x * 256) {
    float s = 0.f;
    for (int r = 0; r < a.ph; ++r) s += a.ddp[idx * a.ph + r];
    a.ddelta[idx] = s;
  }
}

// dA and dD: one workgroup per head; thread k sums parts k, k+256, ... in
// order, then a fixed tree over the threads.
__global__ void __launch_bounds__(256) ssd_bwd_reduce_head_kernel(BwdArgs a) {
  __shared__ float sa[256], sd[256];
  const int h = blockIdx.x;
  const int items = a.batch * a.nblk * a.ph;
  float va = 0.f, vd = 0.f;
  for (int i = threadIdx.x; i < items; i += 256) {
    const size_t o = (size_t)(i / a.ph) * a.Hv + (size_t)h * a.ph + i % a.ph;
    va += a.dAp[o];
    vd += a.dDp[o];
  }
  sa[threadIdx.x] = va;
  sd[threadIdx.x] = vd;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      sa[threadIdx.x] += sa[threadIdx.x + s];
      sd[threadIdx.x] += sd[threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.dA[h] = sa[0];
    if (a.dD) a.dD[h] = sd[0];
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdLayout {
  size_t fwd, yf, Sblk, Eblk, Ep, Dp, dBp, dCp, ddp, dAp, dDp, total;
};

// Pieces of blocks for the adjoint passes: about 2560 (piece, virtual head,
// batch) workgroups (ten per CU), whole blocks each.  The environment
// variable MSS_SSD_BWD_BLOCKS_PER_PIECE, when it holds a positive count,
// overrides the piece length (tuning and tests).
void e_pieces(int64_t batch, int64_t vheads, int64_t nblk, int& npc, int& bpp) {
  const int64_t streams = batch * vheads;
  const int64_t np = std::max<int64_t>(1, std::min<int64_t>((2560 + streams - 1) / streams, nblk));
  bpp = (int)((nblk + np - 1) / np);
  if (const char* e = std::getenv("MSS_SSD_BWD_BLOCKS_PER_PIECE")) {
    const long v = std::strtol(e, nullptr, 10);
    if (v >= 1) bpp = (int)std::min<int64_t>(v, nblk);
  }
  npc = (int)((nblk + bpp - 1) / bpp);
}

// Virtual heads per gradient workgroup: the largest divisor of a group's
// virtual heads that still leaves 8 workgroups per CU (2048 for 256 CUs), or 1.
// More heads per workgroup mean fewer dB/dC parts to write and sum and fewer
// loads of B and C; the workgroups run one at a time per CU.  The environment
// variable MSS_SSD_BWD_HEADS_PER_WG, when it holds a divisor of the group's
// virtual heads, overrides the choice (tuning and tests).
int grad_heads_per_wg(int64_t batch, int64_t nblk, int64_t vheads, int64_t ngroups) {
  const int64_t hvg = vheads / ngroups;
  if (const char* e = std::getenv("MSS_SSD_BWD_HEADS_PER_WG")) {
    const long v = std::strtol(e, nullptr, 10);
    if (v >= 1 && v <= hvg && hvg % v == 0) return (int)v;
  }
  for (int64_t d = hvg; d > 1; --d)
    if (hvg % d == 0 && batch * nblk * ngroups * (hvg / d) >= 2048) return (int)d;
  return 1;
}

BwdLayout bwd_layout(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups,
                     int64_t dstate) {
  const int64_t nblk = (seqlen + kSub - 1) / kSub;
  const int64_t vheads = nheads * (headdim / kP);
  const int64_t chunks = vheads / grad_heads_per_wg(batch, nblk, vheads, ngroups);  // G * cpg
  const size_t f4 = sizeof(float);
  BwdLayout l;
  l.fwd = 0;  // the forward's workspace (its status word first)
  l.yf = align256(ssd_workspace_bytes(batch, seqlen, nheads, headdim, ngroups, dstate, kSub));
  l.Sblk = l.yf + align256((size_t)batch * seqlen * nheads * headdim * f4);
  l.Eblk = l.Sblk + align256((size_t)batch * nblk * nheads * headdim * dstate * f4);
  int npc, bpp;
  e_pieces(batch, vheads, nblk, npc, bpp);
  l.Ep = l.Eblk + align256((size_t)batch * nblk * nheads * headdim * dstate * f4);
  l.Dp = l.Ep + align256((size_t)batch * npc * nheads * headdim * dstate * f4);
  l.dBp = l.Dp + align256((size_t)batch * npc * vheads * f4);
  l.dCp = l.dBp + align256((size_t)batch * seqlen * chunks * dstate * f4);
  l.ddp = l.dCp + align256((size_t)batch * seqlen * chunks * dstate * f4);
  l.dAp = l.ddp + align256((size_t)batch * seqlen * vheads * f4);
  l.dDp = l.dAp + align256((size_t)batch * nblk * vheads * f4);
  l.total = l.dDp + align256((size_t)batch * nblk * vheads * f4);
  return l;
}

unsigned stride_grid(size_t total) {
  return (unsigned)std::max<size_t>(1, std::min<size_t>((total + 255) / 256, 16384));
}

}  // namespace

size_t ssd_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups,
                               int64_t dstate) {
  return bwd_layout(batch, seqlen, nheads, headdim, ngroups, dstate).total;
}

hipError_t launch_ssd_bwd(const SSDBwdParams& p, hipStream_t stream) {
  const BwdLayout l = bwd_layout(p.batch, p.seqlen, p.nheads, p.headdim, p.ngroups, p.dstate);
  char* ws = static_cast<char*>(p.workspace);
  // Pass 1: the forward with 64-step chunks, ungated, keeping every block's state.
  SSDParams f;
  f.x = p.x;
  f.delta = p.delta;
  f.A = p.A;
  f.B = p.B;
  f.C = p.C;
  f.D = p.D;
  f.z = nullptr;
  f.h0 = p.h0;
  f.y = p.z ? reinterpret_cast<float*>(ws + l.yf) : nullptr;  // the ungated y serves dz only
  f.chunk_states = reinterpret_cast<float*>(ws + l.Sblk);
  f.h_last = nullptr;
  f.batch = p.batch;
  f.seqlen = p.seqlen;
  f.nheads = p.nheads;
  f.headdim = p.headdim;
  f.ngroups = p.ngroups;
  f.dstate = p.dstate;
  f.chunk = kSub;
  f.workspace = ws + l.fwd;
  hipError_t err = launch_ssd(f, stream);
  if (err != hipSuccess) return err;

  BwdArgs a;
  a.x = static_cast<const uint16_t*>(p.x);
  a.A = p.A;
  a.B = static_cast<const uint16_t*>(p.B);
  a.C = static_cast<const uint16_t*>(p.C);
  a.D = p.D;
  a.z = static_cast<const uint16_t*>(p.z);
  a.h0 = p.h0;
  a.dy = p.dy;
  a.dh_last = p.dh_last;
  a.dx = p.dx;
  a.dz = p.dz;
  a.ddelta = p.ddelta;
  a.dA = p.dA;
  a.dB = p.dB;
  a.dC = p.dC;
  a.dD = p.dD;
  a.dh0 = p.dh0;
  size_t dl_off, ls_off;
  ssd_delta_rows(p.batch, p.seqlen, p.nheads, p.headdim, kSub, dl_off, ls_off);
  a.dlT = reinterpret_cast<const float*>(ws + l.fwd + dl_off);
  a.lsT = reinterpret_cast<const float*>(ws + l.fwd + ls_off);
  a.yf = reinterpret_cast<const float*>(ws + l.yf);
  a.Sblk = reinterpret_cast<const float*>(ws + l.Sblk);
  a.Eblk = reinterpret_cast<float*>(ws + l.Eblk);
  a.Ep = reinterpret_cast<float*>(ws + l.Ep);
  a.Dp = reinterpret_cast<float*>(ws + l.Dp);
  a.dBp = reinterpret_cast<float*>(ws + l.dBp);
  a.dCp = reinterpret_cast<float*>(ws + l.dCp);
  a.ddp = reinterpret_cast<float*>(ws + l.ddp);
  a.dAp = reinterpret_cast<float*>(ws + l.dAp);
  a.dDp = reinterpret_cast<float*>(ws + l.dDp);
  a.batch = (int)p.batch;
  a.L = (int)p.seqlen;
  a.H = (int)p.nheads;
  a.G = (int)p.ngroups;
  a.P = (int)p.headdim;
  a.ph = (int)(p.headdim / kP);
  a.Hv = a.H * a.ph;
  a.N = (int)p.dstate;
  a.nblk = (int)((p.seqlen + kSub - 1) / kSub);
  a.Lp = a.nblk * kSub;
  a.hpw = grad_heads_per_wg(a.batch, a.nblk, a.Hv, a.G);
  a.cpg = a.Hv / a.G / a.hpw;
  a.Gc = a.G * a.cpg;
  e_pieces(a.batch, a.Hv, a.nblk, a.npc, a.bpp);

  const dim3 pieces((unsigned)a.npc * (unsigned)a.Hv, (unsigned)a.batch);
  hipLaunchKernelGGL(ssd_bwd_piece_kernel<false>, pieces, dim3(256), 0, stream, a);
  const unsigned xb = (unsigned)((16 * a.N + 255) / 256);
  hipLaunchKernelGGL(ssd_bwd_piece_chain_kernel, dim3(xb * (unsigned)a.Hv, (unsigned)a.batch), dim3(256), 0, stream,
                     a);
  hipLaunchKernelGGL(ssd_bwd_piece_kernel<true>, pieces, dim3(256), 0, stream, a);
  hipLaunchKernelGGL(ssd_bwd_grad_kernel, dim3((unsigned)a.nblk * (unsigned)a.Gc, (unsigned)a.batch), dim3(512), 0,
                     stream, a);
  hipLaunchKernelGGL(ssd_bwd_reduce_bc_kernel, dim3(stride_grid((size_t)a.batch * a.L * a.G * (a.N / 4))), dim3(256),
                     0, stream, a);
  hipLaunchKernelGGL(ssd_bwd_reduce_dd_kernel, dim3(stride_grid((size_t)a.batch * a.L * a.H)), dim3(256), 0, stream,
                     a);
  hipLaunchKernelGGL(ssd_bwd_reduce_head_kernel, dim3((unsigned)a.H), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mss
