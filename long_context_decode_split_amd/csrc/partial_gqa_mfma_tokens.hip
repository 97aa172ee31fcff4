// One-wave instances of the matrix-core GQA kernel (gqa_mfma_kernel.hpp) for
// two to four query tokens of an fp8 or MXFP4 cache: every wave takes one
// shard of one (request, KV head) and two tokens of the turn.  Two tokens
// keep 9 accumulator blocks each (36 registers per token), which only fit
// next to the register ring as AGPRs: this file is compiled with the default
// accumulator form (the rest of the kernel's instances keep them in VGPRs).
#include "gqa_mfma_kernel.hpp"

namespace kvd {
namespace {

// One wave per (shard, chunk of two tokens); the chunks of a shard are
// neighbouring waves of one workgroup.  With one chunk every cached byte is
// read once (non-temporal loads); with two the second wave's reads of the
// same rows shortly after the first's hit the caches (plain loads).
template <int KV, bool PAGED>
hipError_t launch_solo_tokens(const PartialArgs& a, hipStream_t stream) {
  PartialArgs as = a;
  as.solo_shards = 1;
  const int nchunks = (a.T + 1) / 2;
  const int64_t waves = (int64_t)a.kvp * a.B * a.Hkv * nchunks;
  const dim3 grid((unsigned)((waves + kWaves - 1) / kWaves));
  if (nchunks == 1)
    hipLaunchKernelGGL((gqa_mfma_kernel<KV, PAGED, true, 2, false, true>), grid, dim3(kThreads), 0, stream, as);
  else
    hipLaunchKernelGGL((gqa_mfma_kernel<KV, PAGED, false, 2, false, true>), grid, dim3(kThreads), 0, stream, as);
  return hipSuccess;
}

}  // namespace

hipError_t launch_gqa_solo_tokens(const PartialArgs& a, hipStream_t stream) {
  if (a.T < 2 || a.T > 4) return hipErrorInvalidValue;
  const bool paged = a.layout == kPaged;
  switch (a.kv_format) {
    case kFP8: return paged ? launch_solo_tokens<kFP8, true>(a, stream) : launch_solo_tokens<kFP8, false>(a, stream);
    case kMXFP4:
      return paged ? launch_solo_tokens<kMXFP4, true>(a, stream) : launch_solo_tokens<kMXFP4, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvd
