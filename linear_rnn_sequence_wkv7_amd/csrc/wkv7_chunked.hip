// Chunk-parallel WKV-7 forward on bf16 matrix cores (placeholder until the
// MFMA kernel lands; the API rejects ALGO_CHUNKED meanwhile).
#include "wkv7_internal.h"

namespace wkv7 {
hipError_t launch_chunked(const Params&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace wkv7
