// Append T new tokens per request to the cache: encode their fp32 K and V
// rows into the cache format and store token t where the cache layout puts
// global position positions[b] + t (the decode step's KV write, or the new
// tokens of a multi-token turn; with the striped and staggered layouts every
// shard takes its share of the new tokens).
//
// Encodings (the cache-format readings shared with the decode kernels):
//  - bf16: round to nearest, ties to even;
//  - fp8 E4M3 (OCP "fn"): y = x / scale in fp32, correctly rounded, with the
//    slab's existing scale, then round to nearest E4M3, ties to even,
//    saturating at +-448 (the NaN code is never produced);
//  - MXFP4 (OCP MX v1.0): per block of 32 elements, E = clamp(floor(log2
//    amax) - 2 + 127, 0, 254) (127 for an all-zero block), elements
//    x * 2^(127 - E) rounded to nearest E2M1, ties to even, saturating at
//    +-6; element 2i in the low nibble of byte i.
// One workgroup of one wave per (request, token, KV head, K or V row); the kernel is
// latency-bound (a few KB per call), so it favours plain code.
#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {
namespace {

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);   // NaN stays NaN
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint8_t e4m3_rne_sat(float y) {
  const uint8_t sign = (uint8_t)((__float_as_uint(y) >> 24) & 0x80u);
  const float a = fabsf(y);
  if (!(a < 448.0f)) return sign | 0x7E;                 // saturate (and inf)
  if (a < 0.015625f) {                                   // below 2^-6: steps of 2^-9
    return sign | (uint8_t)rintf(a * 512.0f);            // 8 is the smallest normal code
  }
  const uint32_t u = __float_as_uint(a);
  int e = (int)(u >> 23) - 127;                          // -6 .. 8
  const uint32_t m = u & 0x7FFFFFu;
  uint32_t mq = (m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20; // 3 mantissa bits, ties to even
  if (mq == 8u) {
    mq = 0u;
    e += 1;
  }
  const int ef = e + 7;
  if (ef > 15 || (ef == 15 && mq > 6u)) return sign | 0x7E;
  return sign | (uint8_t)((ef << 3) | (int)mq);
}

__device__ __forceinline__ uint8_t e2m1_rne_sat(float v) {
  const uint8_t sign = (__float_as_uint(v) >> 31) ? 0x8 : 0x0;
  const float a = fabsf(v);
  uint8_t c;
  if (a <= 0.25f) c = 0;        // 0.25: tie to 0
  else if (a < 0.75f) c = 1;    // 0.5
  else if (a <= 1.25f) c = 2;   // 1.0 (ties 0.75 and 1.25 go here)
  else if (a < 1.75f) c = 3;    // 1.5
  else if (a <= 2.5f) c = 4;    // 2.0 (ties 1.75 and 2.5)
  else if (a < 3.5f) c = 5;     // 3.0
  else if (a <= 5.0f) c = 6;    // 4.0 (ties 3.5 and 5.0)
  else c = 7;                   // 6.0, saturating
  return sign | c;
}

__global__ __launch_bounds__(64) void append_kv_kernel(AppendArgs a) {
  const int rows_per_head = a.v_aliases_k ? 1 : 2;
  int flat = blockIdx.x;
  const int which = flat % rows_per_head;   // 0: K row, 1: V row
  flat /= rows_per_head;
  const int kvh = flat % a.Hkv;
  flat /= a.Hkv;
  const int tok = flat % a.T;
  const int b = flat / a.T;
  const int t = threadIdx.x;

  const int64_t start = a.positions[b];
  if (start < 0) return;                           // the whole request is skipped
  const int64_t pos = start + tok;
  const int64_t bh = (int64_t)b * a.Hkv + kvh;
  int64_t row;
  if (a.layout == kPaged) {
    if (pos >= ((int64_t)a.max_blocks << a.log2_block)) return;
    const int64_t pb = a.block_table[(int64_t)b * a.max_blocks + (pos >> a.log2_block)];
    if (pb < 0 || pb >= a.num_blocks) return;
    row = ((pb * a.Hkv + kvh) << a.log2_block) + (pos & ((1 << a.log2_block) - 1));
  } else {
    int j;
    int64_t r;
    token_home(a.layout, pos, a.kvp, &j, &r);
    if (r >= a.S_max) return;
    const int64_t slab = a.layout == kContiguous ? bh : ((int64_t)j * a.B + b) * a.Hkv + kvh;
    row = slab * a.S_max + r;
  }
  const int D = which ? a.Dv : a.Dqk;
  const float* x = (which ? a.v_new : a.k_new) + (((int64_t)b * a.T + tok) * a.Hkv + kvh) * D;
  uint8_t* data = static_cast<uint8_t*>(which ? a.v : a.k);
  void* scale = which ? a.v_scale : a.k_scale;

  if (a.kv_format == kF32) {
    float* dst = reinterpret_cast<float*>(data) + row * D;
    for (int e = t; e < D; e += 64) dst[e] = x[e];
  } else if (a.kv_format == kBF16) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(data) + row * D;
    for (int e = t; e < D; e += 64) dst[e] = bf16_rne(x[e]);
  } else if (a.kv_format == kFP8) {
    const float s = static_cast<const float*>(scale)[bh];
    uint8_t* dst = data + row * D;
    for (int e = t; e < D; e += 64) dst[e] = e4m3_rne_sat(__fdiv_rn(x[e], s));
  } else {
    uint8_t* dst = data + row * (D / 2);
    uint8_t* sdst = static_cast<uint8_t*>(scale) + row * (D / 32);
    for (int blk = t; blk < D / 32; blk += 64) {
      const float* xb = x + 32 * blk;
      float amax = 0.0f;
      for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(xb[k]));
      int E = 127;
      if (amax > 0.0f) {
        const int fl = ilogbf(amax);                     // floor(log2 amax), exact
        E = fl - 2 + 127;
        E = E < 0 ? 0 : (E > 254 ? 254 : E);
      }
      sdst[blk] = (uint8_t)E;
      for (int k = 0; k < 16; ++k) {
        const uint8_t lo = e2m1_rne_sat(ldexpf(xb[2 * k], 127 - E));
        const uint8_t hi = e2m1_rne_sat(ldexpf(xb[2 * k + 1], 127 - E));
        dst[16 * blk + k] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

}  // namespace

hipError_t launch_append_kv(const AppendArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.B * a.T * a.Hkv * (a.v_aliases_k ? 1 : 2);
  hipLaunchKernelGGL(append_kv_kernel, dim3((unsigned)blocks), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvd
