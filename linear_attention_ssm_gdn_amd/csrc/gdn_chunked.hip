// gdn_chunked.hip -- chunked WY/UT prefill (placeholder until the MFMA kernel lands).
#include "gdn_kernels.h"

namespace gdn {

bool chunked_supported(int, int, int) { return false; }

hipError_t launch_chunked(const ChunkArgs&, int, int, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace gdn
