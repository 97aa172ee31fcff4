// Host-side interface between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvd {

// Arguments of one split-KV partial pass, already validated by api.cpp.
struct PartialArgs {
  const void* q;
  const void* k;
  const void* k_scale;
  const void* v;          // == k when V aliases K
  const void* v_scale;    // == k_scale when V aliases K
  const int32_t* seq_lens;
  float* o_part;
  float* lse_part;
  int32_t B, Hq, Hkv, Dqk, Dv, kvp;
  int32_t T;              // query tokens per request (q [B,T,Hq,Dqk])
  int64_t S_max;
  int32_t q_bf16;         // q is bf16 (else fp32)
  int32_t kv_format;      // KvFormat
  int32_t v_aliases_k;
  float scale_log2;       // sm_scale * log2(e)
  int32_t layout;         // CacheLayout
  // paged layout only
  const int32_t* block_table;   // [B, max_blocks]
  int32_t log2_block;           // block_len = 1 << log2_block
  int32_t max_blocks;
  int64_t num_blocks;
  // set by the launcher of the matrix-core GQA kernel: consecutive shards
  // one wave streams when it takes whole shards (0 otherwise)
  int32_t solo_shards;
};

// Arguments of one append (kvd_append_kv), already validated by api.cpp.
struct AppendArgs {
  const float* k_new;     // [B,T,Hkv,Dqk]
  const float* v_new;     // [B,T,Hkv,Dv]; nullptr when V aliases K
  const int32_t* positions;   // [B]: token t of request b goes to positions[b] + t
  void* k;
  void* k_scale;
  void* v;
  void* v_scale;
  int32_t B, Hkv, Dqk, Dv, kvp;
  int32_t T;              // new tokens per request
  int64_t S_max;
  int32_t kv_format;
  int32_t v_aliases_k;
  int32_t layout;
  const int32_t* block_table;
  int32_t log2_block;
  int32_t max_blocks;
  int64_t num_blocks;
};

// Grid of a partial pass of U work units with T query tokens each (the id
// layout is unit_token's in kvd_device.hpp): U for T = 1, else U rounded up
// to a multiple of 8 units, times T.
inline int64_t unit_token_blocks(int64_t U, int T) { return T == 1 ? U : (U + 7) / 8 * 8 * T; }

// Each family reports whether it handles a problem, then launches it.
bool valu_supports(const PartialArgs& a);
hipError_t launch_partial_valu(const PartialArgs& a, hipStream_t stream);

bool gqa_mfma_supports(const PartialArgs& a);
hipError_t launch_partial_gqa_mfma(const PartialArgs& a, hipStream_t stream);

// One-wave GQA instances for 2 <= T <= 4 query tokens of an fp8 or MXFP4
// cache, one (shard, two-token chunk) per wave (partial_gqa_mfma_tokens.hip).
hipError_t launch_gqa_solo_tokens(const PartialArgs& a, hipStream_t stream);

// Three or four query tokens of an fp8 cache with 16 query heads per KV head:
// one wave per shard unit, the tokens as columns of 32x32 MFMAs
// (partial_gqa_tokens32.hip).
bool gqa_tokens32_supports(const PartialArgs& a);
hipError_t launch_gqa_tokens32(const PartialArgs& a, hipStream_t stream);

bool mla_mfma_supports(const PartialArgs& a);
hipError_t launch_partial_mla_mfma(const PartialArgs& a, hipStream_t stream);

hipError_t launch_append_kv(const AppendArgs& a, hipStream_t stream);

hipError_t launch_lse_merge(int32_t kvp, int64_t rows, int32_t Dv, const float* o_part,
                            const float* lse_part, float* o, float* lse, hipStream_t stream);

}  // namespace kvd
