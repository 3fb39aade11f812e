// Matrix-core chunked prefill (placeholder until the kernels land).
#include "kda_launch.hpp"

namespace kda {
size_t mfma_block_bytes(int, int) { return 0; }
bool mfma_supported(int, int, int) { return false; }
hipError_t launch_prefill_mfma(const PrefillParams &, void *, int, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace kda
