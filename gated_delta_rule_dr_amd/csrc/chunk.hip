// Placeholder until the matrix-core chunk kernel lands: the bf16 d=128 path runs the fp32
// token-by-token kernel.
#include "dr_internal.h"

namespace dr {
hipError_t launch_chunk128(const Problem& p, hipStream_t stream) { return launch_recurrent(p, stream); }
}  // namespace dr
