// Split-KV partial attention for GQA groups on MFMA (to be filled in).
#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {

bool gqa_mfma_supports(const PartialArgs&) { return false; }

hipError_t launch_partial_gqa_mfma(const PartialArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace kvd
