// Launchers of the matrix-core GQA kernel (gqa_mfma_kernel.hpp) for one
// and two query tokens per workgroup and the four-token LDS ring of bf16
// caches.  This file is compiled with the accumulators in VGPRs (the
// occasional vector-ALU rescale then needs no AGPR copies).
#include "gqa_mfma_kernel.hpp"

namespace kvd {

bool gqa_mfma_supports(const PartialArgs& a) {
  if (!a.q_bf16 || a.v_aliases_k) return false;
  if (a.Dqk != kD || a.Dv != kD) return false;
  // groups of up to 16 query heads (fewer fill part of the 16 MFMA columns)
  const int G = a.Hq / a.Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return false;
  return a.kv_format == kBF16 || a.kv_format == kFP8 || a.kv_format == kMXFP4;
}

// Query tokens per workgroup: a single token streams with non-temporal
// loads; two share each decoded tile with their tiles ahead in registers.  A
// bf16 cache, whose tiles are twice as large, runs three or more tokens four
// to a workgroup with the tiles ahead in an LDS ring (measured faster there;
// slower for the fp8 and MXFP4 caches, whose decode work dominates).  The
// chunks of one shard run on one XCD.
int tokens_per_workgroup(int T, int kv) {
  if (T == 1) return 1;
  return (kv == kBF16 && T >= 3) ? 4 : 2;
}

// Shards per wave for the one-wave split (0: the four-wave split): from
// Layout::kSoloWaves shard units on, each wave streams units / kSoloWaves
// consecutive shards, at least one and at most the kStash its LDS slots hold,
// so the pass runs about kSoloWaves long streams.
template <int KV>
int solo_shards(int64_t units) {
  constexpr int64_t W = Layout<KV>::kSoloWaves;
  if (W == 0 || units < W) return 0;
  const int64_t n = units / W;
  return (int)(n < Layout<KV>::kStash ? n : Layout<KV>::kStash);
}

// A one-token instance, with the format's dynamic LDS: the partials stash of
// the one-wave groups, or the reservation that sets the occupancy.
template <int KV, bool PAGED, bool SOLO>
hipError_t launch_one_token(const PartialArgs& a, dim3 grid, hipStream_t stream) {
  auto fn = gqa_mfma_kernel<KV, PAGED, true, 1, false, SOLO>;
  const size_t lds = SOLO ? stash_bytes<KV>() : (size_t)Layout<KV>::kLdsReserve;
  constexpr size_t kPatch = KV == kBF16 ? 0 : (size_t)kWaves * VPatch<KV>::kWaveBytes;   // static V patches
  static_assert(stash_bytes<KV>() + kPatch <= 160 * 1024, "stash and V patches fit the LDS");
  static_assert(sizeof(MergeLds) + Layout<KV>::kLdsReserve + kPatch <= 160 * 1024, "merge, reserve and V patches fit");
  static_assert(Layout<KV>::kWavesPerEu == 1 || 2 * (stash_bytes<KV>() + kPatch) <= 160 * 1024,
                "two workgroups per CU");
  if (lds > 64 * 1024) {
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
  }
  hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, stream, a);
  return hipSuccess;
}

// The four-token instance (bf16 cache, LDS ring of tiles) with NT loads or not.
template <int KV, bool PAGED, bool NT>
hipError_t launch_gqa_ring(const PartialArgs& a, dim3 grid, hipStream_t stream) {
  constexpr size_t kLds = (size_t)kWaves * Ring::kWaveBytes;
  static_assert(kLds >= sizeof(MergeLds) && kLds <= 160 * 1024, "LDS ring budget");
  auto fn = gqa_mfma_kernel<KV, PAGED, NT, 4, true, false>;
  // more than 64 KB of dynamic LDS: raise the kernel's limit once (the
  // initialization of a local static is thread-safe)
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(fn, grid, dim3(kThreads), kLds, stream, a);
  return hipSuccess;
}

// When one token chunk covers all T tokens every cache byte is read once, so
// the loads carry the non-temporal hint as for a single token; with several
// chunks they are plain, and the later chunks of a shard find its rows in L2.
template <int KV, bool PAGED>
hipError_t launch_gqa3(const PartialArgs& a, hipStream_t stream) {
  const int tw = tokens_per_workgroup(a.T, KV);
  const int nchunks = (a.T + tw - 1) / tw;
  const int64_t blocks = unit_token_blocks((int64_t)a.kvp * a.B * a.Hkv, nchunks);
  const dim3 grid((unsigned)blocks), block(kThreads);
  const int64_t units = (int64_t)a.kvp * a.B * a.Hkv;
  const int nsh = tw == 1 ? solo_shards<KV>(units) : 0;
  if (KV == kFP8 && a.T >= 3 && a.T <= 4 && units >= Layout<KV>::kSoloTokenUnits && gqa_tokens32_supports(a)) {
    // one wave per shard unit, all tokens on 32x32 MFMAs
    return launch_gqa_tokens32(a, stream);
  } else if (KV != kBF16 && a.T >= 2 && a.T <= 4 && units >= Layout<KV>::kSoloTokenUnits) {
    // one wave per (shard, two-token chunk)
    return launch_gqa_solo_tokens(a, stream);
  } else if (nsh > 0) {
    PartialArgs as = a;
    as.solo_shards = nsh;
    const int64_t groups = (int64_t)((a.kvp + nsh - 1) / nsh) * a.B * a.Hkv;
    return launch_one_token<KV, PAGED, true>(as, dim3((unsigned)((groups + kWaves - 1) / kWaves)), stream);
  } else if (tw == 1) {
    return launch_one_token<KV, PAGED, false>(a, grid, stream);
  } else if (tw == 2) {
    if (nchunks == 1)
      hipLaunchKernelGGL((gqa_mfma_kernel<KV, PAGED, true, 2, false, false>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((gqa_mfma_kernel<KV, PAGED, false, 2, false, false>), grid, block, 0, stream, a);
  } else if constexpr (KV == kBF16) {
    return nchunks == 1 ? launch_gqa_ring<KV, PAGED, true>(a, grid, stream)
                        : launch_gqa_ring<KV, PAGED, false>(a, grid, stream);
  } else {
    return hipErrorInvalidValue;   // no four-token instance for this format
  }
  return hipSuccess;
}

hipError_t launch_partial_gqa_mfma(const PartialArgs& a, hipStream_t stream) {
  const bool paged = a.layout == kPaged;
  hipError_t e;
  switch (a.kv_format) {
    case kBF16:
      e = paged ? launch_gqa3<kBF16, true>(a, stream) : launch_gqa3<kBF16, false>(a, stream);
      break;
    case kFP8:
      e = paged ? launch_gqa3<kFP8, true>(a, stream) : launch_gqa3<kFP8, false>(a, stream);
      break;
    case kMXFP4:
      e = paged ? launch_gqa3<kMXFP4, true>(a, stream) : launch_gqa3<kMXFP4, false>(a, stream);
      break;
    default:
      return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace kvd
