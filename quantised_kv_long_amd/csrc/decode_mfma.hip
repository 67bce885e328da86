// decode_mfma.hip -- split-KV decode attention on the matrix cores (not yet
// enabled: the dispatcher falls back to the vector-ALU kernel).
#include "kvq_internal.hpp"

namespace kvq {

bool decode_mfma_supports(const DecodeArgs&) { return false; }

hipError_t launch_decode_mfma(const DecodeArgs&, hipStream_t) { return hipErrorInvalidConfiguration; }

}  // namespace kvq
