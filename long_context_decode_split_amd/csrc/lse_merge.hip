// Exact log-sum-exp merge of shard partials.
//
// For each row r (one query head of one request) with kvp shard partials
// (o_j, lse_j): M = max_j lse_j, w_j = exp(lse_j - M) (zero for an empty shard,
// lse_j = -inf), o = sum_j w_j o_j / sum_j w_j, lse = M + ln sum_j w_j.  This is
// the merge each KV-parallel rank runs after the all-to-all in the Helix
// article ("Sharding the sequence instead"), and the exact merge equation of
// the Context Parallelism note (pass-KV section).
//
// One workgroup per row.  Its threads first find M and the weights w_j
// together (kept in LDS), then split the row's work two ways: with n = Dv/4
// float4 columns (at most 256 at a time), thread t owns the 4 output columns
// 4 (t % n) .. + 3 and the shards j = t / n, j + P, j + 2P, ... with
// P = 256 / n; each streams its columns of those shards with 16-byte loads,
// several in flight, and the P partial sums of a column are added in LDS in
// a fixed order.  Every summation order is fixed,
// so results are bitwise reproducible.
#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {
namespace {

constexpr int kMergeThreads = 256;   // four waves (block_reduce assumes it)
constexpr int kMaxKvp = 4096;          // the ABI's limit on kvp

// Sum (or max) of one value per thread over the workgroup, in a fixed order:
// within each wave by DPP row reductions and the row swaps, then the four wave
// results in wave order.  Every thread gets the result.  `red` holds 4 floats.
template <bool MAX>
__device__ float block_reduce(float v, float* red) {
  v = MAX ? rows4_max(row16_max(v)) : rows4_sum(row16_sum(v));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = MAX ? fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))
                      : ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(int kvp, int64_t rows, int Dv,
                                                                  const float* __restrict__ o_part,
                                                                  const float* __restrict__ lse_part,
                                                                  float* __restrict__ o,
                                                                  float* __restrict__ lse) {
  __shared__ float w[kMaxKvp];
  __shared__ float red[kMergeThreads / 64];
  __shared__ float4 part[kMergeThreads];
  const int64_t r = blockIdx.x;
  const int t = threadIdx.x;

  // ---- M = max_j lse_j, w_j = exp(lse_j - M), W = sum_j w_j
  float m = -INFINITY;
  for (int j = t; j < kvp; j += kMergeThreads) m = fmaxf(m, lse_part[(int64_t)j * rows + r]);
  const float M = block_reduce<true>(m, red);
  float s = 0.0f;
  for (int j = t; j < kvp; j += kMergeThreads) {
    const float lj = lse_part[(int64_t)j * rows + r];
    const float wj = (lj == -INFINITY) ? 0.0f : expf(lj - M);
    w[j] = wj;
    s += wj;
  }
  const float W = block_reduce<false>(s, red);   // also orders the w[] writes before the reads

  // ---- o = sum_j w_j o_j / W, in pages of up to 256 float4 columns
  const int cols4 = Dv / 4;
  const int64_t jstride = rows * (int64_t)cols4;  // float4s between shards
  const float inv = (M == -INFINITY) ? 0.0f : 1.0f / W;
  for (int cbase = 0; cbase < cols4; cbase += kMergeThreads) {
    const int ccount = min(cols4 - cbase, kMergeThreads);
    const int P = kMergeThreads / ccount;         // shard subsets
    const int c4 = cbase + t % ccount, sp = t / ccount;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (M != -INFINITY && sp < P) {
      const float4* src = reinterpret_cast<const float4*>(o_part + r * Dv) + c4;
      int j = sp;
      for (; j + 3 * P < kvp; j += 4 * P) {
        const float4 v0 = src[(int64_t)j * jstride];
        const float4 v1 = src[(int64_t)(j + P) * jstride];
        const float4 v2 = src[(int64_t)(j + 2 * P) * jstride];
        const float4 v3 = src[(int64_t)(j + 3 * P) * jstride];
        const float w0 = w[j], w1 = w[j + P], w2 = w[j + 2 * P], w3 = w[j + 3 * P];
        acc.x = fmaf(w3, v3.x, fmaf(w2, v2.x, fmaf(w1, v1.x, fmaf(w0, v0.x, acc.x))));
        acc.y = fmaf(w3, v3.y, fmaf(w2, v2.y, fmaf(w1, v1.y, fmaf(w0, v0.y, acc.y))));
        acc.z = fmaf(w3, v3.z, fmaf(w2, v2.z, fmaf(w1, v1.z, fmaf(w0, v0.z, acc.z))));
        acc.w = fmaf(w3, v3.w, fmaf(w2, v2.w, fmaf(w1, v1.w, fmaf(w0, v0.w, acc.w))));
      }
      for (; j < kvp; j += P) {
        const float4 v = src[(int64_t)j * jstride];
        const float wj = w[j];
        acc.x = fmaf(wj, v.x, acc.x);
        acc.y = fmaf(wj, v.y, acc.y);
        acc.z = fmaf(wj, v.z, acc.z);
        acc.w = fmaf(wj, v.w, acc.w);
      }
    }
    part[t] = acc;
    __syncthreads();
    if (sp == 0) {
      float4 sum = part[t];
      for (int k = 1; k < P; ++k) {
        const float4 v = part[k * ccount + t];
        sum.x += v.x;
        sum.y += v.y;
        sum.z += v.z;
        sum.w += v.w;
      }
      reinterpret_cast<float4*>(o + r * Dv)[c4] =
          make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
    }
    __syncthreads();   // part[] is reused by the next page
  }
  if (t == 0) lse[r] = (M == -INFINITY) ? -INFINITY : M + logf(W);
}

}  // namespace

hipError_t launch_lse_merge(int32_t kvp, int64_t rows, int32_t Dv, const float* o_part,
                            const float* lse_part, float* o, float* lse, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  // host validation guarantees 1 <= kvp <= 4096 and Dv % 4 == 0, Dv >= 4
  if (kvp < 1 || kvp > kMaxKvp || Dv < 4 || Dv % 4 != 0 || rows > 0x7FFFFFFF)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)rows), dim3(kMergeThreads), 0, stream, kvp,
                     rows, Dv, o_part, lse_part, o, lse);
  return hipGetLastError();
}

}  // namespace kvd
