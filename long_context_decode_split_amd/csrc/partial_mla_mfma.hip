// Split-KV partial attention for latent (MLA) heads on MFMA (to be filled in).
#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {

bool mla_mfma_supports(const PartialArgs&) { return false; }

hipError_t launch_partial_mla_mfma(const PartialArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace kvd
