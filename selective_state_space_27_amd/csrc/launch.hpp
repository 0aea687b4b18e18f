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
// workspace (y, h_last and ckpt unused); dstate <= 16.
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

size_t ssd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                           int64_t ngroups, int64_t dstate, int64_t chunk);
hipError_t launch_ssd(const SSDParams& p, hipStream_t stream);

}  // namespace mss
