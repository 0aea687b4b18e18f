// Internal interface between the C-ABI layer (api.cpp) and the kernel files.
// Arguments have already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mss {

struct ScanParams {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;   // nullable
  const void* z;    // nullable
  const float* h0;  // nullable
  void* y;
  float* h_last;    // nullable
  int64_t batch, dim, dstate, seqlen;
  bool bf16;
  bool force_general;
  void* workspace;
  // Where a bounded wait that gives up is reported (cleared at the start of
  // the call): the workspace's first word when null.
  int* status = nullptr;
  float* ckpt = nullptr;  // backward only: states entering every tile, [b*nblocks][ntiles][8][SPW][64]
  // Fused prologue (u = x and delta = delta_raw above): u from the causal
  // 4-tap convolution of x, delta from delta_raw plus bias, optionally softplus.
  bool fused = false;
  const float* conv_w = nullptr;      // [dim][4]
  const float* conv_b = nullptr;      // [dim], nullable
  const float* delta_bias = nullptr;  // [dim], nullable
  bool conv_silu = false;
  bool delta_softplus = false;
};

size_t scan_workspace_bytes(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen);
hipError_t launch_scan(const ScanParams& p, hipStream_t stream);

// Backward of the selective scan: fwd holds the forward's inputs, shape and
// workspace (y, h_last and ckpt unused); dstate <= 32 for launch_scan_bwd.
struct ScanBwdParams {
  ScanParams fwd;
  const void* dy;
  const float* dh_last;  // nullable
  void* du;
  void* ddelta;
  float* dA;
  void* dB;
  void* dC;
  float* dD;             // nullable
  void* dz;              // non-null exactly when fwd.z is
  float* dh0;            // nullable
};

size_t scan_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen);
hipError_t launch_scan_bwd(const ScanBwdParams& p, hipStream_t stream);
// Backward of the scan fed by its prologue (x, delta_raw and the taps and
// biases in place of u and delta); any d_state the scan backward takes.
struct ScanFusedBwdParams {
  const void* x;
  const void* delta_raw;
  const float* conv_w;      // [dim][4]
  const float* conv_b;      // nullable
  const float* delta_bias;  // nullable
  bool conv_silu, softplus;
  const float* A;
  const void* B;
  const void* C;
  const float* D;           // nullable
  const void* z;            // nullable
  const float* h0;          // nullable
  const void* dy;
  const float* dh_last;     // nullable
  void* dx;
  void* ddelta_raw;
  float* dconv_w;
  float* dconv_b;           // nullable
  float* ddelta_bias;       // nullable
  float* dA;
  void* dB;
  void* dC;
  float* dD;                // nullable
  void* dz;                 // non-null exactly when z is
  float* dh0;               // nullable
  int64_t batch, dim, dstate, seqlen;
  bool bf16;
  bool force_general;
  void* workspace;
};

size_t scan_fused_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen);
hipError_t launch_scan_fused_bwd(const ScanFusedBwdParams& p, hipStream_t stream);

// d_state 33..128: the same gradient by slices of 32 states, in fp32.
size_t scan_bwd_wide_workspace_bytes(int64_t batch, int64_t dim, int64_t seqlen);
hipError_t launch_scan_bwd_wide(const ScanBwdParams& p, hipStream_t stream);

struct UpdateParams {
  float* h;
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;  // nullable
  const void* z;   // nullable
  void* y;
  int64_t batch, dim, dstate;
  bool bf16;
};

hipError_t launch_state_update(const UpdateParams& p, hipStream_t stream);

struct SSDParams {
  const void* x;
  const float* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;        // nullable
  const void* z;         // nullable
  const float* h0;       // nullable
  float* y;
  float* chunk_states;   // nullable
  float* h_last;         // nullable
  int64_t batch, seqlen, nheads, headdim, ngroups, dstate, chunk;
  void* workspace;
};

// Mamba-3 state update: trapezoid input when x_prev (and B_prev) are given,
// complex state when theta is.
struct Mamba3Params {
  float* h;               // [b, H, P, N] or [b, H, P, N, 2]
  const void* x;          // [b, H, R, P]
  const void* x_prev;     // nullable
  const float* delta;     // [b, H]
  const float* A;         // [H]
  const float* theta;     // [H, N], nullable
  const void* B;          // [b, G, R, N]
  const void* B_prev;     // nullable
  const void* C;          // [b, G, R, N]
  const float* D;         // [H], nullable
  const void* z;          // [b, H, R, P], nullable
  void* y;                // [b, H, R, P]
  int64_t batch, nheads, headdim, ngroups, dstate, rank;
  bool bf16;
};

hipError_t launch_mamba3_step(const Mamba3Params& p, hipStream_t stream);

size_t ssd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                           int64_t ngroups, int64_t dstate, int64_t chunk);
hipError_t launch_ssd(const SSDParams& p, hipStream_t stream);
// Byte offsets, inside the SSD forward's workspace, of its head-major delta
// rows and their prefix sums inside every 64-step block scaled by A log2(e)
// ([b, H, Lp] fp32 each, Lp = seqlen rounded up to 64).
void ssd_delta_rows(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t chunk, size_t& dlT,
                    size_t& lsT);

// Backward of the SSD layer (dstate <= 128): the forward's inputs, dy and
// dh_last (nullable), and the gradients (dD exactly when D, dz exactly when
// z; dh0 nullable).
struct SSDBwdParams {
  const void* x;
  const float* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;        // nullable
  const void* z;         // nullable
  const float* h0;       // nullable
  const float* dy;
  const float* dh_last;  // nullable
  float* dx;
  float* ddelta;
  float* dA;
  float* dB;
  float* dC;
  float* dD;             // nullable
  float* dz;             // nullable
  float* dh0;            // nullable
  int64_t batch, seqlen, nheads, headdim, ngroups, dstate;
  void* workspace;
};

size_t ssd_bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups,
                               int64_t dstate);
hipError_t launch_ssd_bwd(const SSDBwdParams& p, hipStream_t stream);
// d_state 129..256: the same gradient by two halves of the states.
size_t ssd_bwd_halves_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                                      int64_t ngroups);
hipError_t launch_ssd_bwd_halves(const SSDBwdParams& p, hipStream_t stream);

}  // namespace mss
