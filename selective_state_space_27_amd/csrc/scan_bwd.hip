// Selective scan backward (Mamba-1 selective SSM layer) for gfx950.
//
// What is computed: the gradient of a scalar loss through the forward of
// include/mambascan.h, given dy = dloss/dy and optionally dloss/dh_last.
// Training runs the same layer over whole sequences ("Mamba (deep
// learning)", paragraph on how the model trains and generates; "Mamba-1/2/3
// visual guide" section 2 figure: training and prefill use the parallel
// scan); the gradient is the chain rule applied to the forward recurrence in
// reverse time.  Per (b, d), with dh the gradient of the state after step t
// and a_t = exp(delta_t A):
//   dout = dy*silu(z);  dz = dy*out*silu'(z)          (out = C.h + D*u)
//   dh  += C_t*dout;    dC_t += dout*h_t              (summed over d)
//   dA  += dh*h_{t-1}*a_t*delta_t                     (summed over b and t)
//   ddelta_t = sum_n dh*(h_{t-1}*a_t*A + B_t*u_t)
//   du_t     = sum_n dh*delta_t*B_t + D*dout;  dB_t += dh*delta_t*u_t
//   dh  *= a_t                                        (gradient of h_{t-1})
// and dh0 is dh after step 0.
//
// Mapping on CDNA4 (three launches):
//  1. The forward's state-only kernel (scan.hip) writes the state entering
//     every 16-step tile; it reuses the forward's balanced split, carries and
//     split passes, and the fp32 B/C workspace of bc_transpose_kernel.
//  2. scan_bwd_kernel: one workgroup of 8 waves per CU; the streams (batch
//     row, 64-channel block) are split over them as in the forward's balanced
//     split, each piece run in reverse, the gradient of the state handed from
//     the workgroup holding a stream's end to the one holding its start
//     (relaxed agent-scope atomics, as in the forward).  Lanes are channels and
//     the states are split over the waves as in the forward.  Per tile every wave
//     recomputes its states' 16 steps from the checkpoint into registers, then
//     runs the gradient backwards in 4-step blocks.  Sums over states (for du,
//     ddelta, dz) go through LDS to the threads that own the channel's row
//     segment; sums over the 64 channels (dB, dC) are taken in LDS and written
//     per stream.  Global loads of the next tile but one are issued into fixed
//     register slots while the current tile runs (the tile loop is unrolled by
//     two).
//  3. bwd_reduce_kernel: dB, dC summed over the channel blocks and dA, dD over
//     the batch rows, each in a fixed order (deterministic).
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "scan_layout.hpp"

namespace mss {
namespace {

constexpr int kBwdThreads = kWaves * kLanes;  // 512
constexpr int kInPad = kLanes + 4;            // LDS row stride of the per-tile inputs

struct BwdArgs {
  const void* u;
  const void* delta;
  const float* A;
  const float* D;
  const void* z;
  const void* dy;
  const float* dh_last;
  const float* bc;     // forward B/C workspace (bc_index layout)
  const float* ckpt;   // [streams][ntiles][8][SPW][64] state entering each tile
  void* du;
  void* ddelta;
  void* dz;
  float* dh0;
  float* dbc;          // [streams][2][8*SPW][L]: dB (0) and dC (1) summed over the stream's channels
  float* dA_part;      // [streams][2 pieces][8*SPW][64]
  float* dD_part;      // [streams][2 pieces][64][4]
  float* carry;        // [kMaxBwdWG][8][SPW][64]: dh entering the first tile of range g
  int* flags;          // [kMaxBwdWG] carry ready; [kMaxBwdWG + 1] ticket
  int* err;            // the call's status word (the forward workspace's first word): set when a wait gave up
  int* ticket;
  int batch, dim, dstate, seqlen, ntiles, nblocks, nwg;
  float* hloc;         // split passes: [kMaxBwdWG][8][SPW][64] zero-end gradient at the start of range g's first piece
  float* dsum;         // split passes: [kMaxBwdWG][64][4] partial sums of delta over that piece
  int split;           // carries precomputed by the local pass and the chain (no waits, no publishing);
                       // dA, dD partials per (workgroup, piece) instead of per (stream, part)
};

constexpr int kMaxBwdWG = 512;        // workgroups per launch at most
constexpr int kBwdMaxSpins = 1 << 22;
constexpr int kBwdMinPieceTiles = 8;  // split passes only while pieces keep this many tiles

__device__ __forceinline__ float dsilu(float z) {  // d/dz of z*sigmoid(z)
  const float sg = rcp_fast(1.0f + exp2_fast(-z * kLog2e));
  return sg * (1.0f + z * (1.0f - sg));
}

template <bool BF16, int SPW, bool VEC>
__global__ void __launch_bounds__(kBwdThreads, 2) scan_bwd_kernel(BwdArgs a) {
  using S = BCShape<SPW>;
  constexpr int NV = S::kNV;
  constexpr int Np = kWaves * SPW;  // states padded to the wave split
  constexpr uint32_t es = BF16 ? 2 : 4;
  static_assert(!S::kBlockLayout, "the backward uses the tile B/C layout");
  // Per tile: x, delta, u, dout, dy*silu'(z) by [step][channel] (once a
  // block's gradients are known, x, dout and dy*silu'(z) of its steps are
  // replaced by du, ddelta and dz); per 4-step block: per-wave sums over its
  // states by [wave][step][quantity][channel] and per-lane terms of dB, dC by
  // [wave][state][step][quantity][channel].  Rows padded to 68 floats.
  __shared__ __attribute__((aligned(16))) float s_in[5][kTile][kInPad];
  __shared__ __attribute__((aligned(16))) float s_part[kWaves][4][3][kLanes];
  __shared__ __attribute__((aligned(16))) float s_dbc[kWaves][SPW][4][2][kInPad];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int L = a.seqlen, N = a.dstate, ntiles = a.ntiles;
  const bool has_z = a.z != nullptr;
  const int grp = w >> 2;
  const int io_ch = (threadIdx.x & 255) >> 2, io_blk = threadIdx.x & 3;

  // Logical range index in reverse start order (a ticket): a workgroup waits
  // only for the one holding the next range, which has always started first.
  __shared__ int sh_ticket;
  if (threadIdx.x == 0) sh_ticket = atomicAdd(a.ticket, 1);
  __syncthreads();
  const int g = a.nwg - 1 - sh_ticket;

  // Balanced split as in the forward: range g holds tiles [g W/G, (g+1) W/G)
  // of the concatenated streams.  In the single pass (at least as many
  // streams as workgroups) a stream is cut at most once; in the split passes
  // (fewer streams than workgroups) a range holds at most two pieces.  Run order: the
  // end of its first stream (needs nothing in the single pass, publishes at
  // once), whole streams, then the start of its last stream (waits for range
  // g + 1 in the single pass).
  const int64_t nstreams = (int64_t)a.batch * a.nblocks;
  const int64_t wtot = nstreams * ntiles;
  const int64_t r0 = (int64_t)g * wtot / a.nwg, r1 = (int64_t)(g + 1) * wtot / a.nwg;
  const int s_first = (int)(r0 / ntiles), s_last = (int)((r1 - 1) / ntiles);
  const int off_first = (int)(r0 - (int64_t)s_first * ntiles);
  const int end_last = (int)(r1 - (int64_t)s_last * ntiles);
  const int npieces = s_last - s_first + 1;
  const int npieces_g = npieces;

  // One piece: stream s (batch row, 64-channel block), tiles [tb, te) in
  // reverse.  dh enters at te from dh_last (te == ntiles) or from the next
  // workgroup's carry slot g + 1, and leaves at tb to slot g when tb > 0.
  auto run_piece = [&](int s, int tb, int te, int piece) __attribute__((always_inline)) {
  const int b = s / a.nblocks, cb = s % a.nblocks;
  const int c = cb * kLanes + lane;
  const bool cok = c < a.dim;

  // I/O role: group 0 (waves 0-3) streams u and delta and writes du, ddelta;
  // group 1 (waves 4-7) streams z and dy and writes dz.  A thread owns channel
  // io_ch of the block and 4-step block io_blk of every tile.
  const int c_io = cb * kLanes + io_ch;
  const bool iok = c_io < a.dim;
  const int nch = min(kLanes, a.dim - cb * kLanes);
  const size_t base_el = ((size_t)b * a.dim + (size_t)cb * kLanes) * (size_t)L;
  const uint32_t rows_bytes = (uint32_t)nch * (uint32_t)L * es;
  const uint32_t io_off = (uint32_t)io_ch * (uint32_t)L * es;
  auto rsrc_of = [&](const void* p) {
    return make_rsrc(p != nullptr ? static_cast<const char*>(p) + base_el * es : nullptr, p != nullptr ? rows_bytes : 0u);
  };
  const rsrc_t r_in0 = rsrc_of(grp == 0 ? a.u : a.z);
  const rsrc_t r_in1 = rsrc_of(grp == 0 ? a.delta : a.dy);
  const rsrc_t r_out0 = rsrc_of(grp == 0 ? a.du : (has_z ? a.dz : nullptr));
  const rsrc_t r_out1 = rsrc_of(grp == 0 ? a.ddelta : nullptr);
  const float dskip = (a.D != nullptr && cok) ? a.D[c] : 0.f;  // of the lane's channel

  // Core constants of this lane's channel and this wave's states.
  float Aj[SPW], A2[SPW], dh[SPW], dA[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int n = w * SPW + j;
    const bool ok = cok && n < N;
    Aj[j] = ok ? a.A[(size_t)c * N + n] : 0.f;
    A2[j] = Aj[j] * kLog2e;
    dh[j] = (te == ntiles && ok && a.dh_last != nullptr) ? a.dh_last[((size_t)b * a.dim + c) * N + n] : 0.f;
    dA[j] = 0.f;
  }
  float dD = 0.f;
  if (te < ntiles) {  // the gradient entering at te, from the workgroup holding [te, ...)
    float* carry = a.carry + ((size_t)(g + 1) * kWaves + w) * SPW * kLanes;
    if (!a.split && threadIdx.x == 0) {
      int spins = 0;
      while (__hip_atomic_load(a.flags + g + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
        __builtin_amdgcn_s_sleep(4);
        if (++spins > kBwdMaxSpins) {  // never expected; keeps every wait finite
          __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SPW; ++j)
      dh[j] = __hip_atomic_load(carry + j * kLanes + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  const rsrc_t rbc = make_rsrc(a.bc + bc_index<SPW>(b, w, 0, ntiles, 0, 0, 0),
                               (uint32_t)ntiles * S::kPerTile * (uint32_t)sizeof(float));
  const float* ckpt = a.ckpt + (((size_t)s * ntiles) * kWaves + w) * SPW * kLanes + lane;

  // Register slots of the prefetch (tile k in slot k & 1 relative to the top).
  Raw4<BF16> in0[2], in1[2];
  f32x4 bct[2][NV];
  float hck[2][SPW];
  auto load = [&](int k, int sl) {
    const bool tok = k >= tb;
    const int t = k * kTile + io_blk * 4;
    in0[sl] = load_raw4<BF16, VEC>(r_in0, io_off, t, L, iok && tok);
    in1[sl] = load_raw4<BF16, VEC>(r_in1, io_off, t, L, iok && tok);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const uint32_t off = tok ? (uint32_t)(((size_t)k * NV + v) * 64 + (lane & 15) * 4) * 4u : kOffNone;
      bct[sl][v] = __builtin_bit_cast(f32x4, buf_load_u32x4(rbc, off));
    }
    const int kc = tok ? k : tb;  // (a tile before the piece is never used)
#pragma unroll
    for (int j = 0; j < SPW; ++j) hck[sl][j] = ckpt[((size_t)kc * kWaves * SPW + j) * kLanes];
  };

  auto tile = [&](int k, auto slot_tag) __attribute__((always_inline)) {
    constexpr int Sl = decltype(slot_tag)::value;
    const int t0 = k * kTile;
    // ---- inputs of the tile into LDS ----
    const f32x4 v0 = decode4(in0[Sl]);  // u (group 0) or z (group 1)
    const f32x4 v1 = decode4(in1[Sl]);  // delta or dy
    f32x4 bc_cur[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) bc_cur[v] = bct[Sl][v];
    float hs[SPW];
#pragma unroll
    for (int j = 0; j < SPW; ++j) hs[j] = hck[Sl][j];
    load(k - 2, Sl);  // the slot is free: the tile after next (in reverse)
    if (grp == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s_in[0][io_blk * 4 + i][io_ch] = v1[i] * v0[i];
        s_in[1][io_blk * 4 + i][io_ch] = v1[i];
        s_in[2][io_blk * 4 + i][io_ch] = v0[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s_in[3][io_blk * 4 + i][io_ch] = has_z ? v1[i] * silu(v0[i]) : v1[i];
        s_in[4][io_blk * 4 + i][io_ch] = has_z ? v1[i] * dsilu(v0[i]) : 0.f;
      }
    }
    __syncthreads();

    // ---- states of the 16 steps, from the checkpoint ----
    // Up to 2 states per wave all 16 steps are held in registers.  With 4 or
    // 8, only the state entering each 4-step block is (hb), and the gradient
    // loop recomputes the block's 4 steps from it: 8 x SPW registers instead
    // of 16 x SPW, which keeps the kernel within 256 VGPRs without spilling.
    constexpr bool kReBlk = SPW >= 4;
    constexpr int kHeld = kReBlk ? 4 : kTile;
    auto fwd = [&](int t, int j, float hp) __attribute__((always_inline)) {
      const int blk = t / 4, kk = t % 4, ib = kk * 2 * SPW + j;
      return __builtin_fmaf(exp2_fast(s_in[1][t][lane] * A2[j]), hp,
                            row_bcast_rt(bc_cur[ib / 16][blk], ib % 16) * s_in[0][t][lane]);
    };
    float h[kHeld][SPW];
    float hb[kReBlk ? kBlk : 1][SPW];
    if constexpr (!kReBlk) {
#pragma unroll
      for (int t = 0; t < kTile; ++t) {
#pragma unroll
        for (int j = 0; j < SPW; ++j) h[t][j] = fwd(t, j, t > 0 ? h[t - 1][j] : hs[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < SPW; ++j) hb[0][j] = hs[j];
#pragma unroll
      for (int t = 0; t < kTile - 4; ++t) {
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
          const float hn = fwd(t, j, t % 4 > 0 ? h[t % 4 - 1][j] : hb[t / 4][j]);
          if (t % 4 == 3) hb[t / 4 + 1][j] = hn;
          else h[t % 4][j] = hn;
        }
      }
    }
    // state after step blk*4 + kk, and the one before it
    auto h_at = [&](int blk, int kk, int j) __attribute__((always_inline)) {
      if constexpr (kReBlk) return h[kk][j];
      else return h[blk * 4 + kk][j];
    };
    auto h_before = [&](int blk, int kk, int j) __attribute__((always_inline)) {
      if constexpr (kReBlk) return kk > 0 ? h[kk - 1][j] : hb[blk][j];
      else return blk * 4 + kk > 0 ? h[blk * 4 + kk - 1][j] : hs[j];
    };

    // ---- gradient, 4-step blocks in reverse ----
#pragma unroll
    for (int blk = kBlk - 1; blk >= 0; --blk) {
      if constexpr (kReBlk) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
          for (int j = 0; j < SPW; ++j) h[kk][j] = fwd(blk * 4 + kk, j, kk > 0 ? h[kk - 1][j] : hb[blk][j]);
        }
      }
#pragma unroll
      for (int kk = 3; kk >= 0; --kk) {
        const int t = blk * 4 + kk;
        const float x = s_in[0][t][lane], dl = s_in[1][t][lane], dout = s_in[3][t][lane];
        float sg = 0.f, s1 = 0.f, outp = 0.f;
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
          const int ib = kk * 2 * SPW + j;  // B of state j at step kk
          const int ic = ib + SPW;          // C of state j at step kk
          dh[j] = fmac_row_bcast_rt(dh[j], bc_cur[ic / 16][blk], dout, ic % 16);
          const float hp = h_before(blk, kk, j), ht = h_at(blk, kk, j);
          const float dec = exp2_fast(dl * A2[j]);
          const float ga = dh[j] * hp * dec;
          dA[j] = __builtin_fmaf(ga, dl, dA[j]);
          sg = __builtin_fmaf(ga, Aj[j], sg);
          s1 = fmac_row_bcast_rt(s1, bc_cur[ib / 16][blk], dh[j], ib % 16);
          outp = fmac_row_bcast_rt(outp, bc_cur[ic / 16][blk], ht, ic % 16);
          s_dbc[w][j][kk][0][lane] = dh[j] * x;
          s_dbc[w][j][kk][1][lane] = dout * ht;
          dh[j] *= dec;
        }
        s_part[w][kk][0][lane] = sg;
        s_part[w][kk][1][lane] = s1;
        s_part[w][kk][2][lane] = outp;
      }
      __syncthreads();

      // dB, dC of the block: 2 x Np x 4 columns of 64 channel terms, each summed
      // by kTpc consecutive threads (a fixed order).
      {
        constexpr int kCols = 2 * Np * 4;
        constexpr int kTpc = kBwdThreads / kCols;  // 8, 4, 2, 1 for SPW 1, 2, 4, 8
        constexpr int kLpt = kLanes / kTpc;
        const int col = threadIdx.x / kTpc, part = threadIdx.x % kTpc;
        const int kk = col % 4, n = (col / 4) % Np, q = col / (4 * Np);
        const float* src = &s_dbc[n / SPW][n % SPW][kk][q][part * kLpt];
        float acc = 0.f;
#pragma unroll 4
        for (int i = 0; i < kLpt; i += 4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(src + i);
          acc += (v[0] + v[1]) + (v[2] + v[3]);
        }
#pragma unroll
        for (int m = 1; m < kTpc; m <<= 1) acc += __shfl_xor(acc, m);
        const int t = t0 + blk * 4 + kk;
        if (part == 0 && t < L) a.dbc[(((size_t)s * 2 + q) * Np + n) * (size_t)L + t] = acc;
      }

      // du, ddelta (group 0) and dz (group 1) of this block: thread (channel
      // lane, step w & 3) of its group sums the 8 waves' partials; the results
      // replace inputs nobody reads any more (x, dout, dy*silu'(z)).
      {
        const int t = blk * 4 + (w & 3);
        if (grp == 0) {
          float sgs = 0.f, s1s = 0.f;
#pragma unroll
          for (int wv = 0; wv < kWaves; ++wv) {
            sgs += s_part[wv][w & 3][0][lane];
            s1s += s_part[wv][w & 3][1][lane];
          }
          const float dout = s_in[3][t][lane], uu = s_in[2][t][lane];
          s_in[0][t][lane] = __builtin_fmaf(s1s, s_in[1][t][lane], dskip * dout);  // du = sum dh B delta + D dout
          s_in[3][t][lane] = __builtin_fmaf(s1s, uu, sgs);                         // ddelta = sum dh (B u + h a A)
          dD = __builtin_fmaf(dout, uu, dD);
        } else {
          float outs = 0.f;
#pragma unroll
          for (int wv = 0; wv < kWaves; ++wv) outs += s_part[wv][w & 3][2][lane];
          s_in[4][t][lane] *= __builtin_fmaf(dskip, s_in[2][t][lane], outs);  // dz = dy silu'(z) out
        }
      }
      __syncthreads();
    }

    // Gradients of the tile's row segments: du, ddelta (group 0), dz (group 1).
    {
      f32x4 o0, o1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o0[i] = s_in[grp == 0 ? 0 : 4][io_blk * 4 + i][io_ch];
        o1[i] = s_in[3][io_blk * 4 + i][io_ch];
      }
      store4<BF16, VEC>(r_out0, io_off, t0 + io_blk * 4, L, iok, o0);  // (no dz stream without z: size 0)
      if (grp == 0) store4<BF16, VEC>(r_out1, io_off, t0 + io_blk * 4, L, iok, o1);
    }
    __syncthreads();  // the next tile overwrites s_in
  };

  load(te - 1, 0);
  load(te - 2, 1);
  int k = te - 1;
  for (; k >= tb + 1; k -= 2) {
    tile(k, std::integral_constant<int, 0>{});
    tile(k - 1, std::integral_constant<int, 1>{});
  }
  if (k == tb) tile(tb, std::integral_constant<int, 0>{});

  if (!a.split && tb > 0) {  // publish the gradient entering tile tb for the workgroup holding [.., tb)
    float* carry = a.carry + ((size_t)g * kWaves + w) * SPW * kLanes;
#pragma unroll
    for (int j = 0; j < SPW; ++j)
      __hip_atomic_store(carry + j * kLanes + lane, dh[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the carry stores have completed
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(a.flags + g, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // Partial sums of the piece and the gradient of the initial state.  Slots:
  // per (stream, part) in the single pass (part 0: the piece starting at tile
  // 0, part 1: the piece ending the stream; a whole stream zeroes part 1);
  // per (workgroup, piece) in the split passes (a range holds at most two
  // pieces there; a lone piece zeroes the second slot).
  const int slot = a.split ? g * 2 + piece : s * 2 + (tb == 0 ? 0 : 1);
  const int zslot = a.split ? g * 2 + 1 : s * 2 + 1;
  const bool whole = a.split ? npieces_g == 1 : (tb == 0 && te == ntiles);
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int n = w * SPW + j;
    a.dA_part[((size_t)slot * Np + n) * kLanes + lane] = dA[j];
    if (whole) a.dA_part[((size_t)zslot * Np + n) * kLanes + lane] = 0.f;
    if (tb == 0 && a.dh0 != nullptr && cok && n < N) a.dh0[((size_t)b * a.dim + c) * N + n] = dh[j];
  }
  if (grp == 0) {
    a.dD_part[((size_t)slot * kLanes + lane) * 4 + (w & 3)] = dD;
    if (whole) a.dD_part[((size_t)zslot * kLanes + lane) * 4 + (w & 3)] = 0.f;
  }
  };

  for (int i = 0; i < npieces; ++i) {
    int s, tb, te;
    if (npieces == 1) {
      s = s_first, tb = off_first, te = end_last;
    } else if (i == 0) {
      s = s_first, tb = off_first, te = ntiles;  // end of the first stream
    } else if (i == npieces - 1) {
      s = s_last, tb = 0, te = end_last;         // start of the last stream
    } else {
      s = s_first + i, tb = 0, te = ntiles;      // whole streams
    }
    run_piece(s, tb, te, i);
  }
}

// Split passes, local part: for range g whose first piece starts inside a
// stream, the gradient of the state at that start when the gradient entering
// at the piece's end is zero (only dh += C dout, dh *= a: no states needed),
// and the sum of delta over the piece.  Same thread roles and register
// prefetch as scan_bwd_kernel; two barriers per tile.
template <bool BF16, int SPW, bool VEC>
__global__ void __launch_bounds__(kBwdThreads) scan_bwd_local_kernel(BwdArgs a) {
  using S = BCShape<SPW>;
  constexpr int NV = S::kNV;
  constexpr uint32_t es = BF16 ? 2 : 4;
  __shared__ __attribute__((aligned(16))) float s_dl[kTile][kInPad];
  __shared__ __attribute__((aligned(16))) float s_do[kTile][kInPad];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int L = a.seqlen, N = a.dstate, ntiles = a.ntiles;
  const int grp = w >> 2;
  const int io_ch = (threadIdx.x & 255) >> 2, io_blk = threadIdx.x & 3;
  const int g = blockIdx.x;
  const int64_t nstreams = (int64_t)a.batch * a.nblocks;
  const int64_t wtot = nstreams * ntiles;
  const int64_t r0 = (int64_t)g * wtot / a.nwg, r1 = (int64_t)(g + 1) * wtot / a.nwg;
  const int s = (int)(r0 / ntiles), s_last = (int)((r1 - 1) / ntiles);
  const int tb = (int)(r0 - (int64_t)s * ntiles);
  if (tb == 0) return;  // the range starts a stream: nothing enters from its left (uniform)
  const int te = s_last == s ? (int)(r1 - (int64_t)s_last * ntiles) : ntiles;

  const int b = s / a.nblocks, cb = s % a.nblocks;
  const int c = cb * kLanes + lane;
  const bool cok = c < a.dim;
  const int c_io = cb * kLanes + io_ch;
  const bool iok = c_io < a.dim;
  const bool has_z = a.z != nullptr;
  const int nch = min(kLanes, a.dim - cb * kLanes);
  const size_t base_el = ((size_t)b * a.dim + (size_t)cb * kLanes) * (size_t)L;
  const uint32_t rows_bytes = (uint32_t)nch * (uint32_t)L * es;
  const uint32_t io_off = (uint32_t)io_ch * (uint32_t)L * es;
  auto rsrc_of = [&](const void* p) {
    return make_rsrc(p != nullptr ? static_cast<const char*>(p) + base_el * es : nullptr, p != nullptr ? rows_bytes : 0u);
  };
  const rsrc_t r_in0 = rsrc_of(grp == 0 ? a.delta : a.z);
  const rsrc_t r_in1 = rsrc_of(grp == 0 ? nullptr : a.dy);
  float A2[SPW], dh[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int n = w * SPW + j;
    A2[j] = (cok && n < N) ? a.A[(size_t)c * N + n] * kLog2e : 0.f;
    dh[j] = 0.f;
  }
  float dacc = 0.f;
  const rsrc_t rbc = make_rsrc(a.bc + bc_index<SPW>(b, w, 0, ntiles, 0, 0, 0),
                               (uint32_t)ntiles * S::kPerTile * (uint32_t)sizeof(float));
  Raw4<BF16> in0[2], in1[2];
  f32x4 bct[2][NV];
  auto load = [&](int k, int sl) {
    const bool tok = k >= tb;
    const int t = k * kTile + io_blk * 4;
    in0[sl] = load_raw4<BF16, VEC>(r_in0, io_off, t, L, iok && tok);
    in1[sl] = load_raw4<BF16, VEC>(r_in1, io_off, t, L, iok && tok);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const uint32_t off = tok ? (uint32_t)(((size_t)k * NV + v) * 64 + (lane & 15) * 4) * 4u : kOffNone;
      bct[sl][v] = __builtin_bit_cast(f32x4, buf_load_u32x4(rbc, off));
    }
  };
  auto tile = [&](int k, auto slot_tag) __attribute__((always_inline)) {
    constexpr int Sl = decltype(slot_tag)::value;
    const f32x4 v0 = decode4(in0[Sl]);  // delta (group 0) or z (group 1)
    const f32x4 v1 = decode4(in1[Sl]);  // (unused) or dy
    f32x4 bc_cur[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) bc_cur[v] = bct[Sl][v];
    load(k - 2, Sl);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (grp == 0) s_dl[io_blk * 4 + i][io_ch] = v0[i];
      else s_do[io_blk * 4 + i][io_ch] = has_z ? v1[i] * silu(v0[i]) : v1[i];
    }
    if (grp == 0) dacc += (v0[0] + v0[1]) + (v0[2] + v0[3]);  // zero past L
    __syncthreads();
#pragma unroll
    for (int t = kTile - 1; t >= 0; --t) {
      const int blk = t / 4, kk = t % 4;
      const float dout = s_do[t][lane], dl = s_dl[t][lane];
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int ic = kk * 2 * SPW + j + SPW;  // C of state j at step kk
        dh[j] = fmac_row_bcast_rt(dh[j], bc_cur[ic / 16][blk], dout, ic % 16);
        dh[j] *= exp2_fast(dl * A2[j]);
      }
    }
    __syncthreads();
  };
  load(te - 1, 0);
  load(te - 2, 1);
  int k = te - 1;
  for (; k >= tb + 1; k -= 2) {
    tile(k, std::integral_constant<int, 0>{});
    tile(k - 1, std::integral_constant<int, 1>{});
  }
  if (k == tb) tile(tb, std::integral_constant<int, 0>{});
#pragma unroll
  for (int j = 0; j < SPW; ++j) a.hloc[(((size_t)g * kWaves + w) * SPW + j) * kLanes + lane] = dh[j];
  if (grp == 0) a.dsum[((size_t)g * kLanes + io_ch) * 4 + io_blk] = dacc;
}

// Split passes, chain: for every stream walk its piece starts from right to
// left, g <- hloc + exp2(A log2e sum delta) * g starting from dh_last (or
// zero): the exact gradient at each piece start, written to the carry slot the
// workgroup holding the piece to its left reads.  One thread per (stream,
// state, channel).
template <int SPW>
__global__ void __launch_bounds__(256) bwd_combine_kernel(const float* __restrict__ hloc,
                                                          const float* __restrict__ dsum, const float* __restrict__ A,
                                                          const float* __restrict__ dh_last, float* __restrict__ carry,
                                                          int batch, int dim, int N, int ntiles, int nblocks, int nwg) {
  const int64_t nstreams = (int64_t)batch * nblocks;
  const int Np = kWaves * SPW;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= nstreams * Np * kLanes) return;
  const int c = (int)(idx % kLanes);
  const int n = (int)((idx / kLanes) % Np);
  const int64_t s = idx / ((int64_t)kLanes * Np);
  const int b = (int)(s / nblocks), cg = (int)(s % nblocks) * kLanes + c;
  const bool ok = cg < dim && n < N;
  const float a2 = ok ? A[(size_t)cg * N + n] * kLog2e : 0.f;
  float gr = (ok && dh_last != nullptr) ? dh_last[((size_t)b * dim + cg) * N + n] : 0.f;
  const int64_t wtot = nstreams * ntiles, s0 = s * ntiles, s1 = s0 + ntiles;
  const int w = n / SPW, j = n % SPW;
  for (int gg = (int)min<int64_t>(nwg - 1, s1 * nwg / wtot + 1); gg >= 1; --gg) {
    const int64_t r0 = (int64_t)gg * wtot / nwg;  // start of range gg
    if (r0 >= s1) continue;
    if (r0 <= s0) break;
    const float* ds = dsum + ((size_t)gg * kLanes + c) * 4;
    const float sd = (ds[0] + ds[1]) + (ds[2] + ds[3]);
    const size_t k = (((size_t)gg * kWaves + w) * SPW + j) * kLanes + c;
    gr = __builtin_fmaf(exp2f(a2 * sd), gr, hloc[k]);
    carry[k] = gr;
  }
}

// Clears the backward's carry flags and ticket (the status word was cleared
// by the forward pass of the same call).
__global__ void __launch_bounds__(256) bwd_clear_kernel(int* flags, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) flags[i] = 0;
}

// Partial-sum slots holding stream s's pieces: (s, part 0..1) in the single
// pass; in the split passes (range g, piece 0 or 1) for every range that
// covers s, piece 0 when s is the range's first stream.  Calls f(slot).
template <typename F>
__device__ __forceinline__ void for_stream_slots(int64_t s, int split, int64_t nstreams, int ntiles, int nwg, F&& f) {
  if (!split) {
    f(s * 2);
    f(s * 2 + 1);
    return;
  }
  const int64_t wtot = nstreams * ntiles, s0 = s * ntiles, s1 = s0 + ntiles;
  for (int64_t gg = max<int64_t>(0, s0 * nwg / wtot - 1); gg < nwg; ++gg) {
    const int64_t r0 = gg * wtot / nwg, r1 = (gg + 1) * wtot / nwg;
    if (r1 <= s0) continue;
    if (r0 >= s1) break;
    f(gg * 2 + (r0 / ntiles == s ? 0 : 1));
  }
}

// dB, dC [b, N, L] = sums of the per-stream partials over the channel blocks;
// dA [d, N] and dD [d] = sums over the batch rows and stream pieces; fixed
// order.  One thread per output element; index ranges: dB, then dC, then dA,
// then dD.
template <bool BF16, int SPW>
__global__ void __launch_bounds__(256) bwd_reduce_kernel(const float* __restrict__ dbc, const float* __restrict__ dA_part,
                                                         const float* __restrict__ dD_part, void* dB, void* dC,
                                                         float* __restrict__ dA, float* __restrict__ dD, int batch,
                                                         int dim, int N, int L, int nblocks, int ntiles, int nwg,
                                                         int split) {
  constexpr int Np = kWaves * SPW;
  const int64_t nbc = (int64_t)batch * N * L;
  const int64_t total = 2 * nbc + (int64_t)dim * N + dim;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
  if (idx < 2 * nbc) {
    const int q = (int)(idx / nbc);
    const int64_t r = idx % nbc;
    const int t = (int)(r % L);
    const int n = (int)((r / L) % N);
    const int b = (int)(r / ((int64_t)L * N));
    float acc = 0.f;
    for (int cb = 0; cb < nblocks; ++cb)
      acc += dbc[((((size_t)b * nblocks + cb) * 2 + q) * Np + n) * (size_t)L + t];
    void* out = q == 0 ? dB : dC;
    if (BF16) static_cast<uint16_t*>(out)[r] = f32_to_bf16(acc);
    else static_cast<float*>(out)[r] = acc;
    continue;
  }
  int64_t r = idx - 2 * nbc;
  if (r < (int64_t)dim * N) {
    const int d = (int)(r / N), n = (int)(r % N);
    float acc = 0.f;
    const int64_t nstreams = (int64_t)batch * nblocks;
    for (int b = 0; b < batch; ++b)
      for_stream_slots((int64_t)b * nblocks + d / kLanes, split, nstreams, ntiles, nwg, [&](int64_t sl) {
        acc += dA_part[((size_t)sl * Np + n) * kLanes + d % kLanes];
      });
    dA[r] = acc;
    continue;
  }
  r -= (int64_t)dim * N;
  if (dD != nullptr && r < dim) {
    const int d = (int)r;
    float acc = 0.f;
    const int64_t nstreams = (int64_t)batch * nblocks;
    for (int b = 0; b < batch; ++b)
      for_stream_slots((int64_t)b * nblocks + d / kLanes, split, nstreams, ntiles, nwg, [&](int64_t sl) {
        const float* p = dD_part + ((size_t)sl * kLanes + d % kLanes) * 4;
        acc += (p[0] + p[1]) + (p[2] + p[3]);
      });
    dD[d] = acc;
  }
  }
}

struct BwdLayout {
  size_t fwd, ckpt, dbc, dA, dD, carry, hloc, dsum, flags, total;
};

BwdLayout bwd_layout(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen) {
  const int spw = states_per_wave(dstate);
  const int64_t nstreams = batch * ((dim + kLanes - 1) / kLanes);
  const int64_t np = (int64_t)kWaves * spw;
  BwdLayout l;
  l.fwd = align256(scan_workspace_bytes(batch, dim, dstate, seqlen));
  l.ckpt = align256((size_t)nstreams * num_tiles(seqlen) * np * kLanes * sizeof(float));
  l.dbc = align256((size_t)nstreams * 2 * np * seqlen * sizeof(float));
  const int64_t slots = 2 * std::max<int64_t>(nstreams, kMaxBwdWG);  // per (stream, part) or (range, piece)
  l.dA = align256((size_t)slots * np * kLanes * sizeof(float));
  l.dD = align256((size_t)slots * kLanes * 4 * sizeof(float));
  l.carry = align256((size_t)kMaxBwdWG * np * kLanes * sizeof(float));
  l.hloc = l.carry;
  l.dsum = align256((size_t)kMaxBwdWG * kLanes * 4 * sizeof(float));
  l.flags = align256((size_t)(kMaxBwdWG + 2) * sizeof(int));
  l.total = l.fwd + l.ckpt + l.dbc + l.dA + l.dD + l.carry + l.hloc + l.dsum + l.flags;
  return l;
}

template <bool BF16, int SPW>
hipError_t launch_bwd_typed(const ScanBwdParams& p, hipStream_t stream) {
  const BwdLayout l = bwd_layout(p.fwd.batch, p.fwd.dim, p.fwd.dstate, p.fwd.seqlen);
  char* ws = static_cast<char*>(p.fwd.workspace);
  float* ckpt = reinterpret_cast<float*>(ws + l.fwd);
  float* dbc = reinterpret_cast<float*>(ws + l.fwd + l.ckpt);
  float* dA_part = reinterpret_cast<float*>(ws + l.fwd + l.ckpt + l.dbc);
  float* dD_part = reinterpret_cast<float*>(ws + l.fwd + l.ckpt + l.dbc + l.dA);
  char* tail = ws + l.fwd + l.ckpt + l.dbc + l.dA + l.dD;
  float* carry = reinterpret_cast<float*>(tail);
  float* hloc = reinterpret_cast<float*>(tail + l.carry);
  float* dsum = reinterpret_cast<float*>(tail + l.carry + l.hloc);
  int* flags = reinterpret_cast<int*>(tail + l.carry + l.hloc + l.dsum);

  // 1. forward, state only: the checkpoints (and the B/C workspace at its start)
  ScanParams f = p.fwd;
  f.y = nullptr;
  f.h_last = nullptr;
  f.ckpt = ckpt;
  hipError_t err = launch_scan(f, stream);
  if (err != hipSuccess) return err;

  // 2. backward: the streams' tiles split evenly over one workgroup per CU
  const int nblocks = (int)((p.fwd.dim + kLanes - 1) / kLanes);
  const int64_t nstreams = p.fwd.batch * nblocks;
  int dev = 0, cus = 0;
  err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  const int cap = std::min(std::max(cus, 1), kMaxBwdWG);
  const int64_t ntiles = num_tiles(p.fwd.seqlen);
  // Fewer streams than ~4/5 of the workgroups: cut them over all CUs (local
  // pass, chain, final pass).  The local pass (the adjoint alone) costs a
  // fraction of the final one, so this pays from there on; with fewer streams
  // than workgroups a range holds at most two pieces.
  const bool split = nstreams * 5 < (int64_t)cap * 4 && nstreams * ntiles >= (int64_t)cap * kBwdMinPieceTiles;
  const int nwg = split ? cap : (int)std::min<int64_t>(nstreams, cap);
  hipLaunchKernelGGL(bwd_clear_kernel, dim3(1), dim3(256), 0, stream, flags, kMaxBwdWG + 2);
  err = hipGetLastError();  // the gradient kernel relies on the cleared ticket and flags
  if (err != hipSuccess) return err;
  BwdArgs a;
  a.u = p.fwd.u;
  a.delta = p.fwd.delta;
  a.A = p.fwd.A;
  a.D = p.fwd.D;
  a.z = p.fwd.z;
  a.dy = p.dy;
  a.dh_last = p.dh_last;
  a.bc = reinterpret_cast<const float*>(ws + scan_flags_bytes());
  a.err = reinterpret_cast<int*>(ws);
  a.ckpt = ckpt;
  a.du = p.du;
  a.ddelta = p.ddelta;
  a.dz = p.dz;
  a.dh0 = p.dh0;
  a.dbc = dbc;
  a.dA_part = dA_part;
  a.dD_part = dD_part;
  a.carry = carry;
  a.hloc = hloc;
  a.dsum = dsum;
  a.split = split ? 1 : 0;
  a.flags = flags;
  a.ticket = flags + kMaxBwdWG + 1;
  a.nwg = nwg;
  a.batch = (int)p.fwd.batch;
  a.dim = (int)p.fwd.dim;
  a.dstate = (int)p.fwd.dstate;
  a.seqlen = (int)p.fwd.seqlen;
  a.ntiles = (int)num_tiles(p.fwd.seqlen);
  a.nblocks = nblocks;
  if (split) {
    if (p.fwd.seqlen % 4 == 0)
      hipLaunchKernelGGL((scan_bwd_local_kernel<BF16, SPW, true>), dim3((unsigned)nwg), dim3(kBwdThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((scan_bwd_local_kernel<BF16, SPW, false>), dim3((unsigned)nwg), dim3(kBwdThreads), 0, stream, a);
    const int64_t threads = nstreams * kWaves * SPW * kLanes;
    hipLaunchKernelGGL((bwd_combine_kernel<SPW>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, hloc,
                       dsum, p.fwd.A, p.dh_last, carry, (int)p.fwd.batch, (int)p.fwd.dim, (int)p.fwd.dstate,
                       (int)ntiles, nblocks, nwg);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (p.fwd.seqlen % 4 == 0)
    hipLaunchKernelGGL((scan_bwd_kernel<BF16, SPW, true>), dim3((unsigned)nwg), dim3(kBwdThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((scan_bwd_kernel<BF16, SPW, false>), dim3((unsigned)nwg), dim3(kBwdThreads), 0, stream, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;

  // 3. fixed-order sums
  const int64_t total = 2 * p.fwd.batch * p.fwd.dstate * p.fwd.seqlen + p.fwd.dim * p.fwd.dstate + p.fwd.dim;
  const unsigned rgrid = (unsigned)std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 16384));
  hipLaunchKernelGGL((bwd_reduce_kernel<BF16, SPW>), dim3(rgrid), dim3(256), 0, stream, dbc,
                     dA_part, dD_part, p.dB, p.dC, p.dA, p.dD, (int)p.fwd.batch, (int)p.fwd.dim, (int)p.fwd.dstate,
                     (int)p.fwd.seqlen, nblocks, (int)ntiles, nwg, split ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

size_t scan_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen) {
  return bwd_layout(batch, dim, dstate, seqlen).total;
}

hipError_t launch_scan_bwd(const ScanBwdParams& p, hipStream_t stream) {
  // d_state <= 32 (up to 4 states per wave).
  auto typed = [&](auto bf16_tag) {
    constexpr bool BF16 = decltype(bf16_tag)::value;
    switch (states_per_wave(p.fwd.dstate)) {
      case 1: return launch_bwd_typed<BF16, 1>(p, stream);
      case 2: return launch_bwd_typed<BF16, 2>(p, stream);
      default: return launch_bwd_typed<BF16, 4>(p, stream);
    }
  };
  return p.fwd.bf16 ? typed(std::true_type{}) : typed(std::false_type{});
}

}  // namespace mss
