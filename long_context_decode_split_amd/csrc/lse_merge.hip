// Exact log-sum-exp merge of shard partials.
//
// For each row r (one query head of one request) with kvp shard partials
// (o_j, lse_j): M = max_j lse_j, w_j = exp(lse_j - M) (zero for an empty shard,
// lse_j = -inf), o = sum_j w_j o_j / sum_j w_j, lse = M + ln sum_j w_j.  This is
// the merge each KV-parallel rank runs after the all-to-all in the Helix
// article ("Sharding the sequence instead"), and the exact merge equation of
// the Context Parallelism note (pass-KV section).
//
// A thread owns 4 consecutive output columns of one row; the Dv/4 threads of
// a row each recompute the row's M and sum of weights from the kvp lse values
// (a few hundred bytes, served from cache) and then stream their columns of
// every shard with 16-byte loads.  Shards are visited in ascending order, so
// results are bitwise reproducible.
#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {
namespace {

constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(int kvp, int64_t rows, int Dv,
                                                                  const float* __restrict__ o_part,
                                                                  const float* __restrict__ lse_part,
                                                                  float* __restrict__ o,
                                                                  float* __restrict__ lse) {
  const int cols4 = Dv / 4;
  const int64_t gid = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  const int64_t r = gid / cols4;
  const int c4 = (int)(gid - r * cols4);
  if (r >= rows) return;

  float M = -INFINITY;
  for (int jj = 0; jj < kvp; ++jj) M = fmaxf(M, lse_part[(int64_t)jj * rows + r]);

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.0f;
  if (M != -INFINITY) {
    for (int jj = 0; jj < kvp; ++jj) {
      const float lj = lse_part[(int64_t)jj * rows + r];
      const float w = (lj == -INFINITY) ? 0.0f : expf(lj - M);
      den += w;
      const float4 v = reinterpret_cast<const float4*>(o_part + ((int64_t)jj * rows + r) * Dv)[c4];
      acc.x = fmaf(w, v.x, acc.x);
      acc.y = fmaf(w, v.y, acc.y);
      acc.z = fmaf(w, v.z, acc.z);
      acc.w = fmaf(w, v.w, acc.w);
    }
    const float inv = 1.0f / den;
    acc.x *= inv;
    acc.y *= inv;
    acc.z *= inv;
    acc.w *= inv;
  }
  reinterpret_cast<float4*>(o + r * Dv)[c4] = acc;
  if (c4 == 0) lse[r] = (M == -INFINITY) ? -INFINITY : M + logf(den);
}

}  // namespace

hipError_t launch_lse_merge(int32_t kvp, int64_t rows, int32_t Dv, const float* o_part,
                            const float* lse_part, float* o, float* lse, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t threads = rows * (Dv / 4);
  const int64_t blocks = (threads + kMergeThreads - 1) / kMergeThreads;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)blocks), dim3(kMergeThreads), 0, stream, kvp,
                     rows, Dv, o_part, lse_part, o, lse);
  return hipGetLastError();
}

}  // namespace kvd
