// Mamba-2 SSD chunked layer (placeholder until the MFMA kernels land).
#include "common.hpp"
#include "launch.hpp"

namespace mss {
size_t ssd_workspace_bytes(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t) { return 256; }
hipError_t launch_ssd(const SSDParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace mss
