// Matrix-core (MFMA) paged MLA decode: not built yet; every request falls
// back to the vector-ALU kernel or is rejected.
#include "internal.h"

namespace mla {

bool decode_mfma_supported(int, int, int, int, int) { return false; }

hipError_t launch_decode_mfma(const DecodeArgs&, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace mla
