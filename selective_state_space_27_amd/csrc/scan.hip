// Selective scan forward (Mamba-1 selective SSM layer) for gfx950.
//
// What is computed (per batch b and channel d, see include/mambascan.h):
//   h[n] <- exp(delta*A[d,n]) * h[n] + delta*B[b,n,l]*u      (recurrence)
//   y    <- (sum_n C[b,n,l]*h[n] + D[d]*u) * silu(z)          (readout, skip, gate)
// following the discretised recurrence of "Mamba (deep learning)" (state-space
// paragraph: Abar = exp(Delta*A)) and "Mamba-1/2/3 visual guide" (section 1 SSM
// equation; section 2 selectivity table and block diagram).  The expanded state
// stays in registers (section 2 figure: many steps combined on-chip, only the
// outputs written back).
//
// Mapping on CDNA4.  One workgroup = 16 wave64s working on one block of 64
// channels of one batch row, time in tiles of 16 steps, one barrier per tile:
//   8 core waves: lanes are channels; the d_state states are split across the
//     waves (SPW = ceil(N/8) each), so every wave's sequential chain is 1/8 of
//     the work.  B and C are shared by every channel: each lane loads a few
//     (fp32, pre-arranged by bc_transpose_kernel) and the multiplies take them
//     from lane p of the row with a DPP row broadcast (v_mul_f32_dpp /
//     v_fmac_f32_dpp row_newbcast:p).  Partial readouts go to LDS; wave 0's
//     includes the skip term D*u.
//   4 prologue waves: for tile k+1, x = delta*u, D*u and the decay data into
//     LDS.
//   4 epilogue waves: for tile k-1, the 8 partial readouts summed in a fixed
//     order, gated by silu(z), stored (u is read once, by the prologue).
// Prologue and epilogue threads own one channel and 4 steps of a tile, so the
// four lanes of a channel read or write its 16-step row segment in one
// instruction.  Streams are read with branch-free buffer loads issued three
// tiles ahead into fixed register slots: the loops are unrolled by three so
// nothing in flight is ever copied, which keeps the in-order vmcnt waits from
// draining the prefetch.  Four waves per SIMD give the issue slack a single
// wave (one VALU instruction per 8 cycles at most) does not have.
//
// Decay, chosen per block of 64 channels from A (checked on the device):
//   S4D-real (A[d,n] == (n+1)*A[d,0] in every channel): the prologue computes
//     one r = exp2(delta*A[d,0]*log2 e) per (d,l) and the start power
//     r^(g*SPW+1) of each wave's states; the waves continue the power chain
//     with multiplies.
//   scalar (A[d,n] == A[d,0] in every channel, the Mamba-2 form of A): every
//     state decays by the same r, computed once per (d,l) by the prologue.
//   general: each wave evaluates exp2(delta*A[d,n]*log2 e) per state.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "scan_layout.hpp"

namespace mss {
namespace {

constexpr int kIoWaves = 4;  // prologue waves, and as many epilogue waves
constexpr int kThreads = (kWaves + 2 * kIoWaves) * kLanes;
// LDS quantities per (d,l): x = delta*u, r (or delta), D*u, and the start
// powers of core waves 1..7 (wave 0's is r itself).
constexpr int kQMax = 2 + kWaves;
constexpr int kQDu = 2;  // slot of D*u
constexpr int kPrefetch = 3;       // tiles of global loads in flight

struct ScanArgs {
  const void* u;
  const void* delta;
  const float* A;
  const float* D;
  const void* z;
  const float* h0;
  void* y;
  float* h_last;
  const float* bc;     // B and C per wave and tile, fp32, in the layout bc_index() describes
  const int* decay_mode;  // [nblocks]: kDecayGeneral, kDecayS4D or kDecayScalar
  float* carry;        // [kMaxWG boundaries][8 waves][SPW][64 lanes] state at the end of workgroup g's range
  float* hloc;         // same layout: zero-start end state of the piece ending at boundary g (split pass)
  float* dsum;         // [kMaxWG][64 channels][4]: partial sums of delta over that piece (split pass)
  float* ckpt;         // state-only kernels outside the local pass: [streams][ntiles][8][SPW][64] (nullable)
  int* flags;          // [kMaxWG]: carry of workgroup g ready
  int* err;            // status word of the call: set when a bounded carry wait gave up
  int* ticket;
  int batch, dim, dstate, seqlen, ntiles, nblocks, nwg;
  int force_general;
  int pass;            // kPassSingle, kPassLocal or kPassFinal
  // Fused prologue: u and delta above are x and the raw delta; the prologue
  // waves form u = (silu of) the causal 4-tap convolution of x and
  // delta = (softplus of) delta_raw + bias.
  const float* conv_w;      // [dim][4]
  const float* conv_b;      // [dim] or null
  const float* delta_bias;  // [dim] or null
  int fused, conv_silu, delta_softplus;
};

constexpr float kLn2 = 0.6931471805599453f;

// softplus(v) = log(1 + exp(v)) = max(v, 0) + log1p(exp(-|v|)), with log1p(e)
// taken as log(w) * e / (w - 1), w = 1 + e rounded (exact for the rounding of
// w; e itself when w rounds to 1).
__device__ __forceinline__ float softplus_f(float v) {
  const float e = exp2_fast(-fabsf(v) * kLog2e);
  const float w = 1.0f + e;
  const float l = (w == 1.0f) ? e : __builtin_amdgcn_logf(w) * kLn2 * (e * rcp_fast(w - 1.0f));
  return fmaxf(v, 0.f) + l;
}

// The value of lane q-1 of this lane's quad (lane 0 of a quad gets lane 3's).
__device__ __forceinline__ float quad_prev(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x93, 0xf, 0xf, false));
}

constexpr int kMaxSpins = 1 << 22;

// Workgroups per launch at most (carry slots are per workgroup boundary).
constexpr int kMaxWG = kMaxScanWG;

// Passes.  Single: one launch, each carry handed to the next workgroup through
// a flag.  When there are too few sequences to fill the chip, sequences are
// cut into more pieces than workgroups could hand on in turn, and three
// launches replace the single one: Local (every piece that ends mid-sequence
// runs from a zero state; its end state and the sum of delta over it are
// kept), carry_combine_kernel (chains those along each sequence into the
// exact start state of every piece), Final (every piece runs from its start
// state, all at once).
constexpr int kPassSingle = 0;
constexpr int kPassLocal = 1;
constexpr int kPassFinal = 2;

// Decay modes of a 64-channel block.
constexpr int kDecayGeneral = 0;  // exp2(delta*A[d,n]*log2 e) per state
constexpr int kDecayS4D = 1;      // A[d,n] == (n+1)*A[d,0]: powers of one r per (d,l)
constexpr int kDecayScalar = 2;   // A[d,n] == A[d,0]: one r per (d,l) for every state




// LDS: per buffer, kQMax quantities x kBlk x channels x float4 (4 steps), and
// 8 waves x kBlk x channels x float4 of partial readouts, each (quantity,
// block) row of channels padded to kRowPad 16-byte slots.  The core accesses
// (lane = channel, one 4-step block) are contiguous.  The prologue/epilogue
// accesses have four lanes per channel, one per block (a block row lies 2
// slots further modulo 32 slots), and io_channel() gives every 8, 16 or 32
// consecutive lanes channels whose slots do not meet modulo 128, 256 or 512
// bytes: {c, c+1}, then {c, c+1, c+8, c+9}, then those and +16.
constexpr int kRowPad = kLanes + 2;
constexpr int kQFloats = kQMax * kBlk * kRowPad * 4;
constexpr int kPFloats = kWaves * kBlk * kRowPad * 4;

// Float offset of (quantity q, block blk, channel ch) in a buffer:
// q_lane(blk, ch) + q * q_step.  The part fixed per thread and the constant
// per quantity stay separate, so the constant folds into the LDS
// instruction's offset field.
__device__ __forceinline__ constexpr int q_lane(int blk, int ch) { return (blk * kRowPad + ch) * 4; }
constexpr int q_step = kBlk * kRowPad * 4;

// Channel (0..63 within the block) of prologue/epilogue wave io (0..3), lane
// `lane`; the lane's 4-step block is lane & 3.  Lane bits 2, 5, 3, 4 and the
// wave bits 0, 1 give channel bits 0, 1, 3, 4 and 2, 5.
__device__ __forceinline__ int io_channel(int io, int lane) {
  return ((lane >> 2) & 1) | (((lane >> 5) & 1) << 1) | ((io & 1) << 2) | (((lane >> 3) & 1) << 3) |
         (((lane >> 4) & 1) << 4) | ((io >> 1) << 5);
}

template <bool BF16, int SPW, bool VEC, bool STATE, bool FUSED>
__global__ void __launch_bounds__(kThreads, 1) scan_kernel(ScanArgs a) {
  using S = BCShape<SPW>;
  constexpr int NV = S::kNV;
  constexpr uint32_t es = BF16 ? 2 : 4;
  __shared__ __attribute__((aligned(16))) float qbuf[2][kQFloats];
  __shared__ __attribute__((aligned(16))) float pbuf[2][kPFloats];
  __shared__ int sh_ticket;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave id, uniform
  const bool is_core = w < kWaves;
  const bool is_pro = !is_core && w < kWaves + kIoWaves;
  const int wc = is_core ? w : 0;  // core wave index (states wc*SPW ..)
  const int L = a.seqlen, N = a.dstate;
  const bool has_z = a.z != nullptr;
  // Prologue and epilogue waves: a thread owns channel io_ch of the block and
  // the 4-step block io_blk of every tile, so four consecutive lanes cover one
  // channel's 16 steps and each global access instruction moves 16 whole row
  // segments.
  const int io = is_core ? 0 : (w - kWaves) % kIoWaves;
  const int io_ch = io_channel(io, lane);
  const int io_blk = lane & 3;
  const int p16 = lane & 15;
  const int ntiles = a.ntiles;
  const uint32_t io_off = (uint32_t)io_ch * (uint32_t)L * es;
  const int io_lds = q_lane(io_blk, io_ch);  // this I/O thread's LDS slot within a quantity's rows
  float h[SPW];

  // Logical workgroup id in start order (a ticket), so the workgroup a carry
  // is waited for has always started before the one that waits.  The split
  // passes never wait and use the launch index.
  if (a.pass == kPassSingle) {
    if (threadIdx.x == 0) sh_ticket = atomicAdd(a.ticket, 1);
    __syncthreads();
  }
  const int wg_id = a.pass == kPassSingle ? sh_ticket : (int)blockIdx.x;

  // One piece of work: stream s (batch row, 64-channel block), tiles [tb, te).
  // The carry into it is slot wg_id - 1 (the end of the previous workgroup's
  // range), the carry out of it slot wg_id.
  auto run_piece = [&](int s, int tb, int te, bool carry_in, bool carry_out) __attribute__((always_inline)) {
    const int b = s / a.nblocks, cb = s % a.nblocks;
    const int c = cb * kLanes + lane;     // channel of this lane in the core
    const bool cok = c < a.dim;
    const int c_io = cb * kLanes + io_ch;  // channel of this thread's I/O items
    const bool iok = c_io < a.dim;
    const int mode = a.force_general ? kDecayGeneral : a.decay_mode[cb];

    // Descriptors over this block's rows [b, cb*64 .. +nch, 0..L).
    const int nch = min(kLanes, a.dim - cb * kLanes);
    const size_t base_el = ((size_t)b * a.dim + (size_t)cb * kLanes) * (size_t)L;
    const uint32_t rows_bytes = (uint32_t)nch * (uint32_t)L * es;
    const rsrc_t ru_d = make_rsrc(static_cast<const char*>(a.u) + base_el * es, rows_bytes);
    const rsrc_t rd_d = make_rsrc(static_cast<const char*>(a.delta) + base_el * es, rows_bytes);
    const rsrc_t rz_d =
        make_rsrc(has_z ? static_cast<const char*>(a.z) + base_el * es : nullptr, has_z ? rows_bytes : 0u);
    const rsrc_t ry_d = make_rsrc(static_cast<char*>(a.y) + base_el * es, rows_bytes);
    const rsrc_t rbc = make_rsrc(a.bc + bc_index<SPW>(b, wc, 0, ntiles, 0, 0, 0),
                                 (uint32_t)ntiles * S::kPerTile * (uint32_t)sizeof(float));

    // Per-thread constants: the prologue channel's A[., 0], the epilogue
    // channel's D, the core channel's A row for this wave's states.
    const float a20 = (is_pro && iok) ? a.A[(size_t)c_io * N] * kLog2e : 0.f;
    const float dskip = (is_pro && a.D != nullptr && iok) ? a.D[c_io] : 0.f;
    // Fused prologue: this prologue channel's taps and biases.
    f32x4 cw = {0.f, 0.f, 0.f, 0.f};
    float cbias = 0.f, dbias = 0.f;
    if (FUSED && is_pro && iok) {
      cw = *reinterpret_cast<const f32x4*>(a.conv_w + (size_t)c_io * 4);
      cbias = a.conv_b != nullptr ? a.conv_b[c_io] : 0.f;
      dbias = a.delta_bias != nullptr ? a.delta_bias[c_io] : 0.f;
    }
    // The core channel's A row for this wave's states (general decay only),
    // loaded inside that mode's loop so the other modes do not keep it live.
    auto load_a2 = [&](float* A2) {
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int n = wc * SPW + j;
        A2[j] = (is_core && cok && n < N) ? a.A[(size_t)c * N + n] * kLog2e : 0.f;
      }
    };

    // Initial state: zero in the local pass; for a piece that continues a
    // sequence, the carry at the end of the previous workgroup's range
    // (published by that workgroup, or chained by carry_combine_kernel before
    // the final pass); else h0 (or zero).
    //
    // The hand-off uses relaxed agent-scope atomics only: on this multi-die
    // part they are coherent loads and stores past the per-die L2, whereas
    // acquire/release at agent scope would also write back or invalidate the
    // whole L2 of the die (on every poll of the flag), stalling every other
    // workgroup there.  Order comes from the producer waiting for its carry
    // stores to complete before it sets the flag, and from the consumer
    // issuing its carry loads only after it has seen the flag.
    const size_t slot_in = ((size_t)(wg_id - 1) * kWaves + wc) * SPW * kLanes;
    const size_t slot_out = ((size_t)wg_id * kWaves + wc) * SPW * kLanes;
    if (STATE && a.pass == kPassLocal) {
#pragma unroll
      for (int j = 0; j < SPW; ++j) h[j] = 0.f;
    } else if (carry_in) {
      float* carry = a.carry + slot_in;
      if (a.pass == kPassSingle && threadIdx.x == 0) {
        int spins = 0;
        while (__hip_atomic_load(a.flags + wg_id - 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
          __builtin_amdgcn_s_sleep(4);
          if (++spins > kMaxSpins) {  // never expected; keeps every wait finite, reported through err
            __hip_atomic_store(a.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
      }
      __syncthreads();
      if (is_core) {
#pragma unroll
        for (int j = 0; j < SPW; ++j)
          h[j] = __hip_atomic_load(carry + j * kLanes + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else if (is_core) {
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int n = wc * SPW + j;
        h[j] = (a.h0 != nullptr && cok && n < N) ? a.h0[((size_t)b * a.dim + c) * N + n] : 0.f;
      }
    }

    // ---- core waves: this wave's SPW states of the block's 64 channels ----
    auto core_run = [&](auto mode_tag) __attribute__((always_inline)) {
      constexpr int M = decltype(mode_tag)::value;
      constexpr bool S4D = M == kDecayS4D;
      // B/C registers.  Tile layout (SPW <= 8): a ring of three tiles (tile t
      // in slot (t - tb) % 3) loaded two tiles ahead, value i of block blk in
      // component blk of bct[slot][i / 16].  Block layout (SPW == 16, whose
      // per-tile share would not fit): a ring of four 4-step blocks (block blk
      // of any tile in slot blk) loaded three blocks ahead, value i in
      // component (i / 16) % 4 of bcb[blk][i / 64].
      constexpr bool kBlkBC = S::kBlockLayout;
      constexpr int kRing = kBlkBC ? 1 : kPrefetch;
      float A2[M == kDecayGeneral ? SPW : 1];
      if constexpr (M == kDecayGeneral) load_a2(A2);
      f32x4 bct[kRing][NV];
      f32x4 bcb[kBlk][kBlkBC ? NV / 4 : 1];
      auto load_bc = [&](int tile, f32x4* dst) {
        const uint32_t tile_ok = tile < te ? 1u : 0u;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const uint32_t off = tile_ok ? (uint32_t)(((size_t)tile * NV + v) * 64 + p16 * 4) * 4u : kOffNone;
          dst[v] = __builtin_bit_cast(f32x4, buf_load_u32x4(rbc, off));
        }
      };
      auto load_bc_blk = [&](int tile, int blk, f32x4* dst) {
        const uint32_t tile_ok = tile < te ? 1u : 0u;
#pragma unroll
        for (int vq = 0; vq < NV / 4; ++vq) {
          const uint32_t off =
              tile_ok ? (uint32_t)((((size_t)tile * kBlk + blk) * (NV / 4) + vq) * 64 + p16 * 4) * 4u : kOffNone;
          dst[vq] = __builtin_bit_cast(f32x4, buf_load_u32x4(rbc, off));
        }
      };
      if constexpr (kBlkBC) {
        load_bc_blk(tb, 0, bcb[0]);
        load_bc_blk(tb, 1, bcb[1]);
        load_bc_blk(tb, 2, bcb[2]);
      } else {
        load_bc(tb, bct[0]);
        load_bc(tb + 1, bct[1]);
      }

      // One tile: x, the decay (S4D: r) and the start power of the four
      // blocks come from qbuf (read all up front when the registers allow);
      // partial readouts go to pbuf, wave 0's starting from D*u.  Steps at or past L need no guard: their
      // delta, u and B read as zero, so the decay is exp2(0) = 1 and the input
      // term 0, and the update leaves h unchanged.
      constexpr int kAhead = SPW <= 4 ? kBlk : 1;
      const int sp_slot = wc == 0 ? 1 : 2 + wc;  // start power r^(wc*SPW+1): r itself for wave 0
      // W0: 1 = wave 0, whose readout starts from D*u, 0 = another wave (a
      // separate copy of the loop, so the other waves keep a plain multiply
      // for their first term); 2 = either, wave 0 adding D*u to its block's
      // partials afterwards (SPW >= 4, whose registers do not allow two
      // copies of the loop).
      auto core_tile = [&](auto w0_tag, int buf, int k, const f32x4* bc_cur) {
        constexpr int W0 = decltype(w0_tag)::value;
        const float* q = qbuf[buf];
        float* pp = pbuf[buf];
        f32x4 xvs[kAhead], rvs[kAhead], svs[kAhead];
        auto read_blk = [&](int blk, int i) {
          const float* qb = q + q_lane(blk, lane);
          xvs[i] = *reinterpret_cast<const f32x4*>(&qb[0]);
          rvs[i] = *reinterpret_cast<const f32x4*>(&qb[q_step]);
          if constexpr (S4D) svs[i] = *reinterpret_cast<const f32x4*>(&qb[sp_slot * q_step]);
          else svs[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        };
        if constexpr (kAhead == kBlk) {
#pragma unroll
          for (int blk = 0; blk < kBlk; ++blk) read_blk(blk, blk);
        }
#pragma unroll
        for (int blk = 0; blk < kBlk; ++blk) {
          if constexpr (kBlkBC) {  // block blk + 3: this tile's last block, or the next tile's
            constexpr int kNext = 3;
            const int nb = (blk + kNext) % kBlk;
            load_bc_blk(blk + kNext < kBlk ? k : k + 1, nb, bcb[nb]);
          }
          // B/C value i of this block (a register and its row position).
          auto bcv = [&](int i) -> float {
            if constexpr (kBlkBC) return bcb[blk][(i / 16) / 4][(i / 16) % 4];
            else return bc_cur[i / 16][blk];
          };
          if constexpr (kAhead == 1) read_blk(blk, 0);
          const int i = kAhead == kBlk ? blk : 0;
          const f32x4 xv = xvs[i], rv = rvs[i], sv = svs[i];
          f32x4 duv;
          if constexpr (W0 == 1 && !STATE) duv = *reinterpret_cast<const f32x4*>(&q[q_lane(blk, lane) + kQDu * q_step]);
          f32x4 part;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const float x = xv[kk];
            const float r = rv[kk];  // r (S4D, scalar) or delta (general)
            float p = 0.f;
            float dec = sv[kk];
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
              const int ib = kk * 2 * SPW + j;  // B of state j at step kk
              const int ic = ib + SPW;          // C of state j at step kk
              if constexpr (S4D) {
                if (j > 0) dec *= r;
              } else if constexpr (M == kDecayScalar) {
                dec = r;
              } else {
                dec = exp2_fast(r * A2[j]);
              }
              const float bx = row_bcast_rt(bcv(ib), ib % 16) * x;
              h[j] = __builtin_fmaf(dec, h[j], bx);
              // Without the readout nothing but the end state uses h, and the
              // optimiser then restructures the tile into far more live
              // values than registers; an empty asm per step keeps each h.
              if constexpr (STATE) asm volatile("" : "+v"(h[j]));
              if constexpr (!STATE) {  // the state-only passes need no readout
                if (j == 0) {
                  if constexpr (W0 == 1) p = fmac_row_bcast_rt(duv[kk], bcv(ic), h[j], ic % 16);
                  else p = row_bcast_rt(bcv(ic), ic % 16) * h[j];
                } else
                  p = fmac_row_bcast_rt(p, bcv(ic), h[j], ic % 16);
              }
            }
            part[kk] = p;
          }
          if constexpr (W0 == 2 && !STATE) {
            if (wc == 0) part += *reinterpret_cast<const f32x4*>(&q[q_lane(blk, lane) + kQDu * q_step]);
          }
          if constexpr (!STATE) *reinterpret_cast<f32x4*>(&pp[q_lane(blk, lane) + wc * q_step]) = part;
        }
      };

      __syncthreads();  // the prologue of tile tb is in qbuf
      // Checkpoint pass: the state entering every tile, for the backward.
      auto checkpoint = [&](int k) {
        if constexpr (STATE) {
          if (a.ckpt != nullptr && a.pass != kPassLocal) {
            float* cp = a.ckpt + ((((size_t)s * ntiles + k) * kWaves + wc) * SPW) * kLanes + lane;
#pragma unroll
            for (int j = 0; j < SPW; ++j) cp[j * kLanes] = h[j];
          }
        }
      };
      if constexpr (kBlkBC) {
        for (int k = tb; k < te; ++k) {
          checkpoint(k);
          core_tile(std::integral_constant<int, 2>{}, k & 1, k, nullptr);
          __syncthreads();
        }
      } else {
        auto step = [&](auto slot_tag, int k) {
          constexpr int Sl = decltype(slot_tag)::value;
          constexpr int S2 = (Sl + 2) % kPrefetch;
          load_bc(k + 2, bct[S2]);  // past the last tile: reads zeros, unused
          checkpoint(k);
          if constexpr (SPW > 2) core_tile(std::integral_constant<int, 2>{}, k & 1, k, bct[Sl]);
          else if (wc == 0) core_tile(std::integral_constant<int, 1>{}, k & 1, k, bct[Sl]);
          else core_tile(std::integral_constant<int, 0>{}, k & 1, k, bct[Sl]);
          __syncthreads();
        };
        int k = tb;
        for (; k + kPrefetch <= te; k += kPrefetch) {
          step(std::integral_constant<int, 0>{}, k);
          step(std::integral_constant<int, 1>{}, k + 1);
          step(std::integral_constant<int, 2>{}, k + 2);
        }
        if (k < te) step(std::integral_constant<int, 0>{}, k);
        if (k + 1 < te) step(std::integral_constant<int, 1>{}, k + 1);
      }
    };

    // ---- prologue waves prepare tile k+1 and epilogue waves finish tile k-1
    // while the core runs tile k ----
    auto io_run = [&](auto mode_tag, auto pro_tag, auto gate_tag) __attribute__((always_inline)) {
      constexpr int M = decltype(mode_tag)::value;
      constexpr bool PRO = decltype(pro_tag)::value;
      constexpr bool GATE = decltype(gate_tag)::value;  // epilogue: z given (a copy of the loop per case)
      if constexpr (STATE && !PRO) {  // no outputs in the state-only passes: keep the barrier count only
        for (int k = tb; k <= te; ++k) __syncthreads();
        return;
      }
      float dacc = 0.f;  // local pass: sum of delta over this thread's steps of the piece
      // Rings of three slots: (u, delta) for the prologue hold tile t in slot
      // (t - tb) % 3 and are loaded three steps ahead; z for the epilogue
      // holds tile t in slot (t - tb + 2) % 3, also three steps ahead.
      // In every step both rings consume and refill the same compile-time
      // slot, and the loop (unrolled by 3) never copies a register whose load
      // is in flight nor branches around a load.
      Raw4<BF16> pu[kPrefetch], pd[kPrefetch], ez[kPrefetch];
      auto load_pro = [&](int tile, int slot) {
        const int t = tile * kTile + io_blk * 4;
        const bool ok = iok && tile >= tb && tile < te;
        pu[slot] = load_raw4<BF16, VEC>(ru_d, io_off, t, L, ok);
        pd[slot] = load_raw4<BF16, VEC>(rd_d, io_off, t, L, ok);
      };
      auto load_epi = [&](int tile, int slot) {
        if constexpr (!GATE) return;
        const int t = tile * kTile + io_blk * 4;
        const bool ok = iok && tile >= tb && tile < te;
        ez[slot] = load_raw4<BF16, VEC>(rz_d, io_off, t, L, ok);
      };

      // Fused prologue: the convolution reads the three steps before this
      // thread's 4-step block from lane q-1 of its quad (the same channel's
      // previous block); block 0 keeps them from lane 3 of the previous tile
      // (hx), or, at the start of a piece, loads them (zeros before step 0).
      float hx1 = 0.f, hx2 = 0.f, hx3 = 0.f;
      if constexpr (PRO && FUSED) {
        if (tb > 0) {
          const f32x4 v = decode4(load_raw4<BF16, VEC>(ru_d, io_off, tb * kTile - 4, L, iok));
          hx1 = v[1], hx2 = v[2], hx3 = v[3];
        }
      }
      auto fuse = [&](f32x4& uu, f32x4& dd, int tile) {
        const float p1 = quad_prev(uu[1]), p2 = quad_prev(uu[2]), p3 = quad_prev(uu[3]);
        const bool first = io_blk == 0;
        const float x1 = first ? hx1 : p1, x2 = first ? hx2 : p2, x3 = first ? hx3 : p3;
        hx1 = p1, hx2 = p2, hx3 = p3;  // lane 3's last steps, for block 0 of the next tile
        const float xs[7] = {x1, x2, x3, uu[0], uu[1], uu[2], uu[3]};
        f32x4 c, v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float acc = cbias;
#pragma unroll
          for (int k = 0; k < 4; ++k) acc = __builtin_fmaf(cw[k], xs[i + k], acc);  // tap k: step t - 3 + k
          c[i] = a.conv_silu ? silu(acc) : acc;
          const float vi = dd[i] + dbias;
          v[i] = a.delta_softplus ? softplus_f(vi) : vi;
        }
        // Steps past the piece (the tile after its last, prepared but never
        // run, whose delta would still enter the local pass's sum of delta)
        // and at or past L must leave the state alone: delta 0, u 0.
        if (tile >= te || (tile + 1) * kTile > L) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool in = tile < te && tile * kTile + io_blk * 4 + i < L;
            c[i] = in ? c[i] : 0.f;
            v[i] = in ? v[i] : 0.f;
          }
        }
        uu = c;
        dd = v;
      };

      // Prologue of one tile from ring slot `slot` into qbuf[buf]: x = delta*u,
      // then r = exp2(delta*A0*log2 e) and the start powers r^(w*SPW+1) (S4D),
      // r alone (scalar) or delta itself (general decay).
      auto prologue = [&](int buf, int slot, int tile, auto&& refill) {
        f32x4 uu = decode4(pu[slot]);
        f32x4 dd = decode4(pd[slot]);
        if constexpr (FUSED) fuse(uu, dd, tile);
        if constexpr (STATE) dacc += (dd[0] + dd[1]) + (dd[2] + dd[3]);  // zero past the piece and past L
        refill();  // the slot's registers are free: issue its next load now
        float* q = qbuf[buf] + io_lds;  // quantity k of this thread's (channel, block) at q[k * q_step]
        *reinterpret_cast<f32x4*>(&q[0]) = dd * uu;
        if constexpr (!STATE) *reinterpret_cast<f32x4*>(&q[kQDu * q_step]) = dskip * uu;
        if constexpr (M == kDecayScalar) {
          f32x4 r;
#pragma unroll
          for (int i = 0; i < 4; ++i) r[i] = exp2_fast(dd[i] * a20);
          *reinterpret_cast<f32x4*>(&q[q_step]) = r;
        } else if constexpr (M == kDecayS4D) {
          f32x4 r;
#pragma unroll
          for (int i = 0; i < 4; ++i) r[i] = exp2_fast(dd[i] * a20);
          *reinterpret_cast<f32x4*>(&q[q_step]) = r;
          f32x4 stp = r;  // r^SPW
#pragma unroll
          for (int j = 1; j < SPW; ++j) stp = stp * r;
          f32x4 sp = r;   // r^(wave*SPW + 1), slot 2 + wave (wave 0 uses r)
#pragma unroll
          for (int wv = 1; wv < kWaves; ++wv) {
            sp = sp * stp;
            *reinterpret_cast<f32x4*>(&q[(2 + wv) * q_step]) = sp;
          }
        } else {
          *reinterpret_cast<f32x4*>(&q[q_step]) = dd;
        }
      };

      // Epilogue of tile `tile`: the 8 partial readouts from pbuf[buf] (D*u
      // is in wave 0's) summed in a fixed order, gated by silu(z); stores only
      // inside the piece.
      auto epilogue = [&](int buf, int slot, int tile, auto&& refill) {
        const f32x4 zz = GATE ? decode4(ez[slot]) : f32x4{0.f, 0.f, 0.f, 0.f};
        refill();  // the slot's registers are free: issue its next load now
        const float* pp = pbuf[buf] + io_lds;
        f32x4 acc = *reinterpret_cast<const f32x4*>(&pp[0]);
#pragma unroll
        for (int wv = 1; wv < kWaves; ++wv) acc += *reinterpret_cast<const f32x4*>(&pp[wv * q_step]);
        f32x4 out;
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = GATE ? acc[i] * silu(zz[i]) : acc[i];
        const bool ok = iok && tile >= tb && tile < te;
        store4<BF16, VEC>(ry_d, io_off, tile * kTile + io_blk * 4, L, ok, out);
      };

      if constexpr (PRO) {
#pragma unroll
        for (int sl = 0; sl < kPrefetch; ++sl) load_pro(tb + sl, sl);
        prologue(tb & 1, 0, tb, [&] { load_pro(tb + kPrefetch, 0); });
      } else {
        load_epi(tb - 1, 1);  // (no such tile: zeros, stores masked)
        load_epi(tb, 2);
        load_epi(tb + 1, 0);
      }
      __syncthreads();  // the prologue of tile tb is in qbuf

      auto step = [&](auto slot_tag, int k) {
        constexpr int Sl = decltype(slot_tag)::value;
        constexpr int S1 = (Sl + 1) % kPrefetch;
        const int buf = k & 1;
        if constexpr (PRO)  // tile k+1 into the buffer the core is not reading
          prologue(buf ^ 1, S1, k + 1, [&] { load_pro(k + 1 + kPrefetch, S1); });
        else  // tile k-1: its partial readouts are complete since the last barrier
          epilogue(buf ^ 1, S1, k - 1, [&] { load_epi(k + 2, S1); });
        __syncthreads();
      };
      int k = tb;
      for (; k + kPrefetch <= te; k += kPrefetch) {
        step(std::integral_constant<int, 0>{}, k);
        step(std::integral_constant<int, 1>{}, k + 1);
        step(std::integral_constant<int, 2>{}, k + 2);
      }
      if (k < te) step(std::integral_constant<int, 0>{}, k);
      if (k + 1 < te) step(std::integral_constant<int, 1>{}, k + 1);
      if constexpr (STATE && PRO) {
        if (a.pass == kPassLocal) a.dsum[((size_t)wg_id * kLanes + io_ch) * 4 + io_blk] = dacc;
      }
      // The last tile's partial readouts are complete after the last barrier;
      // its epilogue ring slot is (te - tb + 1) % 3.
      if constexpr (!PRO) {
        const int ph = (te - tb) % kPrefetch;
        const int lb = (te - 1) & 1;
        auto none = [] {};
        if (ph == 0) epilogue(lb, 1, te - 1, none);
        else if (ph == 1) epilogue(lb, 2, te - 1, none);
        else epilogue(lb, 0, te - 1, none);
      }
    };

    using G = std::integral_constant<int, kDecayGeneral>;
    using S4 = std::integral_constant<int, kDecayS4D>;
    using SC = std::integral_constant<int, kDecayScalar>;
    if (is_core) {
      if (mode == kDecayS4D) core_run(S4{});
      else if (mode == kDecayScalar) core_run(SC{});
      else core_run(G{});
    } else if (is_pro) {
      if (mode == kDecayS4D) io_run(S4{}, std::true_type{}, std::false_type{});
      else if (mode == kDecayScalar) io_run(SC{}, std::true_type{}, std::false_type{});
      else io_run(G{}, std::true_type{}, std::false_type{});
    } else {
      // the epilogue is the same for every decay
      if (has_z) io_run(G{}, std::false_type{}, std::true_type{});
      else io_run(G{}, std::false_type{}, std::false_type{});
    }

    if (STATE && a.pass == kPassLocal) {  // the zero-start end state, for carry_combine_kernel (a later launch)
      if (is_core) {
#pragma unroll
        for (int j = 0; j < SPW; ++j) a.hloc[slot_out + j * kLanes + lane] = h[j];
      }
    } else if (carry_out && a.pass == kPassSingle) {  // publish the state after tile te-1
      if (is_core) {
        float* carry = a.carry + slot_out;
#pragma unroll
        for (int j = 0; j < SPW; ++j)
          __hip_atomic_store(carry + j * kLanes + lane, h[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the carry stores have completed
      }
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_store(a.flags + wg_id, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!STATE && is_core && te == ntiles && a.h_last != nullptr && cok) {
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const int n = wc * SPW + j;
        if (n < N) a.h_last[((size_t)b * a.dim + c) * N + n] = h[j];
      }
    }
  };

  // Balanced split: workgroup g owns tiles [g*W/G, (g+1)*W/G) of the
  // concatenation of all streams (W = streams * ntiles, G = workgroups).  In
  // the single pass there are at least as many streams as workgroups, so every
  // range spans a stream end and consists of: the tail of its first stream
  // (which continues the state the previous workgroup reached), whole streams,
  // and the head of its last stream (whose end state the next workgroup
  // continues from).  The head is run first and its state published at once;
  // the tail is run last.  In the split passes a range may also lie inside one
  // stream; the local pass runs only the piece that ends mid-stream.
  const int64_t nstreams = (int64_t)a.batch * a.nblocks;
  const int64_t wtot = nstreams * ntiles;
  const int64_t r0 = (int64_t)wg_id * wtot / a.nwg, r1 = (int64_t)(wg_id + 1) * wtot / a.nwg;
  const int s_first = (int)(r0 / ntiles), s_last = (int)((r1 - 1) / ntiles);
  const int off_first = (int)(r0 - (int64_t)s_first * ntiles);
  const int end_last = (int)(r1 - (int64_t)s_last * ntiles);
  // Pieces in run order (one call site keeps a single inlined copy of the loops).
  const int npieces = s_last - s_first + 1;
  for (int i = 0; i < npieces; ++i) {
    int s, tb, te;
    if (npieces == 1) {
      s = s_first, tb = off_first, te = end_last;
    } else if (i == 0) {
      s = s_last, tb = 0, te = end_last;         // head of the last stream
    } else if (i == npieces - 1) {
      s = s_first, tb = off_first, te = ntiles;  // tail of the first stream
    } else {
      s = s_first + i, tb = 0, te = ntiles;      // whole streams
    }
    if (STATE && a.pass == kPassLocal && te == ntiles) continue;
    run_piece(s, tb, te, tb > 0, te < ntiles);
  }
}

// Split passes, between the local and the final pass: for every stream, walk
// its piece boundaries in order and chain h <- exp(A*sum(delta)) * h + hloc
// (the piece's decay over all its steps times the state entering it, plus its
// zero-start end state), starting from h0 (or zero); the result is the exact
// start state of the next piece, written to its carry slot.  One thread per
// (stream, state, channel).
template <int SPW>
__global__ void __launch_bounds__(256) carry_combine_kernel(const float* __restrict__ hloc,
                                                            const float* __restrict__ dsum,
                                                            const float* __restrict__ A, const float* __restrict__ h0,
                                                            float* __restrict__ carry, int batch, int dim, int N,
                                                            int ntiles, int nblocks, int nwg) {
  const int64_t nstreams = (int64_t)batch * nblocks;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int Np = kWaves * SPW;  // states padded to the wave split
  if (idx >= nstreams * Np * kLanes) return;
  const int c = (int)(idx % kLanes);
  const int n = (int)((idx / kLanes) % Np);
  const int64_t s = idx / ((int64_t)kLanes * Np);
  const int b = (int)(s / nblocks), cg = (int)(s % nblocks) * kLanes + c;
  const bool ok = cg < dim && n < N;
  const float a2 = ok ? A[(size_t)cg * N + n] * kLog2e : 0.f;
  float h = (ok && h0 != nullptr) ? h0[((size_t)b * dim + cg) * N + n] : 0.f;
  const int64_t wtot = nstreams * ntiles, s0 = s * ntiles, s1 = s0 + ntiles;
  const int w = n / SPW, j = n % SPW;
  for (int g = (int)max<int64_t>(0, s0 * nwg / wtot - 1); g < nwg - 1; ++g) {
    const int64_t r1 = (int64_t)(g + 1) * wtot / nwg;  // end of workgroup g's range
    if (r1 <= s0) continue;
    if (r1 >= s1) break;
    const float* ds = dsum + ((size_t)g * kLanes + c) * 4;
    const float sd = (ds[0] + ds[1]) + (ds[2] + ds[3]);
    const size_t k = (((size_t)g * kWaves + w) * SPW + j) * kLanes + c;
    h = __builtin_fmaf(exp2f(a2 * sd), h, hloc[k]);
    carry[k] = h;
  }
}

// B, C [batch, N, L] (bf16 or fp32) -> fp32 workspace in the bc_index layout,
// zero for n >= N, l >= L and unused row positions.  Every loop strides over
// the whole grid, so a capped grid covers any size.  The same launch clears
// the flags block (ticket, carry flags) and the call's status word (the
// block's first word, or the caller's), and picks each 64-channel
// block's decay mode (one wave per block, comparing exactly in fp32):
// kDecayScalar when A[d,n] == A[d,0] for every channel d of the block, else
// kDecayS4D when A[d,n] == (n+1)*A[d,0] for every channel, else kDecayGeneral.
template <bool BF16, int SPW>
__global__ void __launch_bounds__(256) bc_transpose_kernel(const void* __restrict__ B, const void* __restrict__ C,
                                                           float* __restrict__ out, int batch, int N, int L,
                                                           int ntiles, int* __restrict__ flags, int nflags,
                                                           const float* __restrict__ A, int* __restrict__ mode_out,
                                                           int dim, int nblocks, int* __restrict__ status) {
  using S = BCShape<SPW>;
  const size_t stride = (size_t)gridDim.x * blockDim.x;  // a multiple of 64: whole waves
  const size_t idx0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (size_t i = idx0; i < (size_t)nflags; i += stride) flags[i] = 0;
  if (idx0 == 0) *status = 0;
  for (size_t wave = idx0 / kLanes; wave < (size_t)nblocks; wave += stride / kLanes) {
    const int c = (int)wave * kLanes + (int)(idx0 % kLanes);
    bool s4d = true, scalar = true;
    if (c < dim) {
      const float a0 = A[(size_t)c * N];
      for (int n = 1; n < N; ++n) {
        const float an = A[(size_t)c * N + n];
        s4d = s4d && (an == (float)(n + 1) * a0);
        scalar = scalar && (an == a0);
      }
    }
    const bool all_scalar = __all(scalar), all_s4d = __all(s4d);
    if (idx0 % kLanes == 0) mode_out[wave] = all_scalar ? kDecayScalar : all_s4d ? kDecayS4D : kDecayGeneral;
  }
  const size_t total = (size_t)batch * kWaves * ntiles * S::kPerTile;
  for (size_t idx = idx0; idx < total; idx += stride) {
    int blk, p, v;
    size_t rest;
    if constexpr (S::kBlockLayout) {
      p = (int)((idx / 4) % 16);
      v = (int)((idx / 64) % (S::kNV / 4)) * 4 + (int)(idx % 4);
      rest = idx / (64 * (S::kNV / 4));
      blk = (int)(rest % kBlk);
      rest /= kBlk;
    } else {
      blk = (int)(idx % 4);
      p = (int)((idx / 4) % 16);
      rest = idx / 64;
      v = (int)(rest % S::kNV);
      rest /= S::kNV;
    }
    const int tile = (int)(rest % ntiles);
    rest /= ntiles;
    const int g = (int)(rest % kWaves);
    const int b = (int)(rest / kWaves);
    const int i = v * 16 + p;
    float val = 0.f;
    if (i < S::kPerBlk) {
      const int kk = i / (2 * SPW), qn = i % (2 * SPW);
      const int l = tile * kTile + blk * 4 + kk;
      const bool isC = qn >= SPW;
      const int n = g * SPW + (isC ? qn - SPW : qn);
      if (n < N && l < L) {
        const size_t off = ((size_t)b * N + n) * L + l;
        const void* src = isC ? C : B;
        val = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(src)[off]) : static_cast<const float*>(src)[off];
      }
    }
    out[idx] = val;
  }
}

// Grid of the one-dimensional helper kernels: enough 256-thread workgroups
// for `items`, at most kMaxHelperGrid (their loops stride over the grid), so
// the launch stays far below the 2^32 work-items of a dispatch.
constexpr size_t kMaxHelperGrid = 16384;
inline unsigned helper_grid(size_t items) {
  return (unsigned)std::max<size_t>(1, std::min<size_t>((items + 255) / 256, kMaxHelperGrid));
}

size_t carry_floats(int spw) { return (size_t)kMaxWG * kWaves * spw * kLanes; }  // also the hloc size
size_t dsum_floats() { return (size_t)kMaxWG * kLanes * 4; }
size_t flag_ints() { return scan_flags_bytes() / sizeof(int); }

// Sequences are cut into pieces for the split passes when there are at most
// half as many streams as workgroups and each piece still has this many tiles.
constexpr int kMinPieceTiles = 8;

template <bool BF16, int SPW>
hipError_t launch_typed(const ScanParams& p, hipStream_t stream) {
  const int64_t ntiles = num_tiles(p.seqlen);
  const int nblocks = (int)((p.dim + kLanes - 1) / kLanes);
  char* ws = static_cast<char*>(p.workspace);
  int* flags = reinterpret_cast<int*>(ws);
  size_t off = scan_flags_bytes();
  float* bc = reinterpret_cast<float*>(ws + off);
  const size_t nbc = bc_floats(SPW, p.batch, p.seqlen);
  off += align256(nbc * sizeof(float));
  int* mode = reinterpret_cast<int*>(ws + off);
  off += align256((size_t)nblocks * sizeof(int));
  float* carry = reinterpret_cast<float*>(ws + off);
  off += align256(carry_floats(SPW) * sizeof(float));
  float* hloc = reinterpret_cast<float*>(ws + off);
  off += align256(carry_floats(SPW) * sizeof(float));
  float* dsum = reinterpret_cast<float*>(ws + off);
  const int64_t nstreams = p.batch * nblocks;

  hipLaunchKernelGGL((bc_transpose_kernel<BF16, SPW>), dim3(helper_grid(std::max<size_t>(nbc, (size_t)nblocks * kLanes))),
                     dim3(256), 0, stream, p.B, p.C, bc, (int)p.batch, (int)p.dstate, (int)p.seqlen, (int)ntiles,
                     flags, (int)flag_ints(), p.A, mode, (int)p.dim, nblocks, p.status ? p.status : flags);
  hipError_t err = hipGetLastError();  // the scan relies on the cleared ticket and flags
  if (err != hipSuccess) return err;

  ScanArgs a;
  a.u = p.u;
  a.delta = p.delta;
  a.A = p.A;
  a.D = p.D;
  a.z = p.z;
  a.h0 = p.h0;
  a.y = p.y;
  a.h_last = p.h_last;
  a.bc = bc;
  a.decay_mode = mode;
  a.batch = (int)p.batch;
  a.dim = (int)p.dim;
  a.dstate = (int)p.dstate;
  a.seqlen = (int)p.seqlen;
  a.ntiles = (int)ntiles;
  a.carry = carry;
  a.hloc = hloc;
  a.dsum = dsum;
  a.ckpt = p.ckpt;
  a.err = p.status ? p.status : flags;
  a.ticket = flags + 1;
  a.flags = flags + 2;
  a.nblocks = nblocks;
  a.force_general = p.force_general ? 1 : 0;
  a.fused = p.fused ? 1 : 0;
  a.conv_w = p.conv_w;
  a.conv_b = p.conv_b;
  a.delta_bias = p.delta_bias;
  a.conv_silu = p.conv_silu ? 1 : 0;
  a.delta_softplus = p.delta_softplus ? 1 : 0;
  // One workgroup per compute unit at most (the kernel's LDS allows one), so
  // the balanced split covers the chip in a single wave of workgroups.
  int dev = 0, cus = 0;
  err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  const int cap = std::min(std::max(cus, 1), kMaxWG);
  const bool split = nstreams * 2 <= cap && nstreams * ntiles >= (int64_t)cap * kMinPieceTiles;
  a.nwg = split ? cap : (int)std::min<int64_t>(nstreams, cap);
  const dim3 grid((unsigned)a.nwg);
  // With a checkpoint buffer (for the backward) every pass runs state-only.
  auto run = [&](auto state_tag) {
    constexpr bool STATE = decltype(state_tag)::value;
    const bool vec = p.seqlen % 4 == 0;
    if (p.fused) {
      if (vec) hipLaunchKernelGGL((scan_kernel<BF16, SPW, true, STATE, true>), grid, dim3(kThreads), 0, stream, a);
      else hipLaunchKernelGGL((scan_kernel<BF16, SPW, false, STATE, true>), grid, dim3(kThreads), 0, stream, a);
    } else {
      if (vec) hipLaunchKernelGGL((scan_kernel<BF16, SPW, true, STATE, false>), grid, dim3(kThreads), 0, stream, a);
      else hipLaunchKernelGGL((scan_kernel<BF16, SPW, false, STATE, false>), grid, dim3(kThreads), 0, stream, a);
    }
  };
  if (!split) {
    a.pass = kPassSingle;
    if (p.ckpt != nullptr) run(std::true_type{});
    else run(std::false_type{});
  } else {
    a.pass = kPassLocal;
    run(std::true_type{});
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    // nstreams <= cap / 2 here: at most 256 * 8 * 16 * 64 threads
    const int64_t threads = nstreams * kWaves * SPW * kLanes;
    hipLaunchKernelGGL((carry_combine_kernel<SPW>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                       hloc, dsum, p.A, p.h0, carry, (int)p.batch, (int)p.dim, (int)p.dstate, (int)ntiles, nblocks,
                       a.nwg);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    a.pass = kPassFinal;
    if (p.ckpt != nullptr) run(std::true_type{});
    else run(std::false_type{});
  }
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_dtype(const ScanParams& p, hipStream_t stream) {
  switch (states_per_wave(p.dstate)) {
    case 1: return launch_typed<BF16, 1>(p, stream);
    case 2: return launch_typed<BF16, 2>(p, stream);
    case 4: return launch_typed<BF16, 4>(p, stream);
    case 8: return launch_typed<BF16, 8>(p, stream);
    default: return launch_typed<BF16, 16>(p, stream);
  }
}

}  // namespace

size_t scan_workspace_bytes(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen) {
  const int64_t nblocks = (dim + kLanes - 1) / kLanes;
  const int spw = states_per_wave(dstate);
  return scan_flags_bytes() + align256(bc_floats(spw, batch, seqlen) * sizeof(float)) +
         align256((size_t)nblocks * sizeof(int)) + 2 * align256(carry_floats(spw) * sizeof(float)) +
         align256(dsum_floats() * sizeof(float));
}

hipError_t launch_scan(const ScanParams& p, hipStream_t stream) {
  return p.bf16 ? launch_dtype<true>(p, stream) : launch_dtype<false>(p, stream);
}

}  // namespace mss
