// decode_mfma.hip — matrix-core (MFMA) variant of the paged decode kernel.  Not enabled yet: the
// vector-ALU kernel serves every configuration.
#include "pa_kernels.h"

namespace pa {

bool decode_mfma_supports(const DecodeArgs &) { return false; }

hipError_t launch_decode_mfma(const DecodeArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
