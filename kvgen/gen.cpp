// Seeded, counter-based synthetic input generator for split-KV decode attention.
//
// This file produces the bytes that both the GPU library and the CPU oracle
// read: query and KV values drawn from N(0,1), rounded to fp32 / bf16, or
// encoded to OCP fp8 E4M3 (one fp32 scale per slab) or OCP MXFP4 (E2M1
// elements with an E8M0 scale per 32 contiguous elements), plus integer
// sequence lengths.  It holds none of the attention arithmetic and none of the
// decoding that the kernels or the oracle perform: it only writes encoded
// inputs.
//
// Random stream.  Element i of stream (seed, stream) is a deterministic
// function of (seed, stream, i) alone, so any slice of a tensor can be
// regenerated without producing the rest, in any order and on any number of
// threads:
//   base      = splitmix64_mix(seed * GOLDEN ^ stream * STREAM_MUL)
//   r(c)      = splitmix64_mix(base + (c + 1) * GOLDEN)          (SplitMix64,
//               Steele, Lea & Flood, OOPSLA 2014: output c of a generator whose
//               state starts at base)
//   pair p    : u1 = ((r(2p) >> 11) + 1) * 2^-53  in (0, 1]
//               u2 =  (r(2p+1) >> 11)     * 2^-53  in [0, 1)
//   Box-Muller (1958): rad = sqrt(-2 ln u1), z(2p) = rad cos(2 pi u2),
//                                            z(2p+1) = rad sin(2 pi u2).
// The variates are computed in double precision with IEEE basic operations
// only (ln, cos and sin are series written out below; no libm calls), then
// rounded (RNE).
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <thread>
#include <vector>
#include <algorithm>

namespace {

constexpr uint64_t GOLDEN = 0x9E3779B97F4A7C15ull;
constexpr uint64_t STREAM_MUL = 0xD1B54A32D192ED03ull;

inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

inline uint64_t stream_base(uint64_t seed, uint64_t stream) {
  return mix64(seed * GOLDEN ^ stream * STREAM_MUL);
}

inline uint64_t draw(uint64_t base, uint64_t c) { return mix64(base + (c + 1) * GOLDEN); }

constexpr double INV_2_53 = 1.0 / 9007199254740992.0;

// ln(x) for x in (0, 1], from IEEE basic operations only (so the stream is the
// same on every x86-64 host, whatever libm it links): x = m * 2^e with m in
// [sqrt(1/2), sqrt(2)), ln m = 2 atanh(s), s = (m - 1)/(m + 1), |s| < 0.172,
// summed as the odd series 2 (s + s^3/3 + ... + s^25/25) (truncation < 1e-21).
inline double ln_unit(double x) {
  uint64_t bits;
  std::memcpy(&bits, &x, 8);
  int e = (int)((bits >> 52) & 0x7FF) - 1023;
  uint64_t mb = (bits & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull;
  double m;
  std::memcpy(&m, &mb, 8);                      // m in [1, 2)
  if (m > 1.4142135623730951) { m *= 0.5; e += 1; }
  double sv = (m - 1.0) / (m + 1.0);
  double s2 = sv * sv;
  // 1/25, 1/23, ..., 1/3, 1
  static constexpr double C[13] = {1.0 / 25, 1.0 / 23, 1.0 / 21, 1.0 / 19, 1.0 / 17, 1.0 / 15,
                                   1.0 / 13, 1.0 / 11, 1.0 / 9,  1.0 / 7,  1.0 / 5,  1.0 / 3, 1.0};
  double poly = C[0];
  for (int k = 1; k < 13; ++k) poly = poly * s2 + C[k];
  const double LN2_HI = 6.93147180369123816490e-01, LN2_LO = 1.90821492927058770002e-10;
  return (double)e * LN2_HI + ((double)e * LN2_LO + 2.0 * sv * poly);
}

// (cos, sin) of 2 pi u for u in [0, 1): 4u = q + r with q = round(4u), r in
// [-1/2, 1/2], phi = r pi/2 in [-pi/4, pi/4]; Taylor series of sin and cos of
// phi to degree 21/22 (truncation < 1e-22); the quadrant q rotates the pair.
inline void cos_sin_2pi(double u, double* c, double* s) {
  double t = 4.0 * u;
  double q = std::nearbyint(t);
  double phi = (t - q) * 1.5707963267948966;
  double p2 = phi * phi;
  // sin(phi) = phi * sum_k (-p2)^k / (2k+1)!, cos(phi) = sum_k (-p2)^k / (2k)!,
  // k = 0..10, evaluated by Horner from the highest term.
  static constexpr double SC[11] = {
      1.0 / 51090942171709440000.0, -1.0 / 121645100408832000.0, 1.0 / 355687428096000.0,
      -1.0 / 1307674368000.0, 1.0 / 6227020800.0, -1.0 / 39916800.0, 1.0 / 362880.0,
      -1.0 / 5040.0, 1.0 / 120.0, -1.0 / 6.0, 1.0};
  static constexpr double CC[11] = {
      1.0 / 2432902008176640000.0, -1.0 / 6402373705728000.0, 1.0 / 20922789888000.0,
      -1.0 / 87178291200.0, 1.0 / 479001600.0, -1.0 / 3628800.0, 1.0 / 40320.0,
      -1.0 / 720.0, 1.0 / 24.0, -1.0 / 2.0, 1.0};
  double sp = SC[0], cp = CC[0];
  for (int k = 1; k < 11; ++k) {
    sp = sp * p2 + SC[k];
    cp = cp * p2 + CC[k];
  }
  sp *= phi;
  int quad = ((int)q) & 3;
  double cc = cp, ss = sp;
  if (quad == 1) { cc = -sp; ss = cp; }
  else if (quad == 2) { cc = -cp; ss = -sp; }
  else if (quad == 3) { cc = sp; ss = -cp; }
  *c = cc;
  *s = ss;
}

// Both variates of Box-Muller pair p.
inline void normal_pair(uint64_t base, uint64_t p, double* z0, double* z1) {
  double u1 = (double)((draw(base, 2 * p) >> 11) + 1) * INV_2_53;
  double u2 = (double)(draw(base, 2 * p + 1) >> 11) * INV_2_53;
  double rad = std::sqrt(-2.0 * ln_unit(u1));
  double c, s;
  cos_sin_2pi(u2, &c, &s);
  *z0 = rad * c;
  *z1 = rad * s;
}

// Fill out[0..count) with variates start..start+count-1 (as double).
template <class Sink>
void normals_range(uint64_t base, uint64_t start, uint64_t count, Sink sink) {
  uint64_t i = start, end = start + count;
  while (i < end) {
    double z0, z1;
    uint64_t p = i >> 1;
    normal_pair(base, p, &z0, &z1);
    if ((i & 1) == 0) {
      sink(i - start, z0);
      ++i;
      if (i < end) { sink(i - start, z1); ++i; }
    } else {
      sink(i - start, z1);
      ++i;
    }
  }
}

// Run fn(lo, hi) over [0, n) split into contiguous pieces on nthreads threads.
template <class Fn>
void parallel_for(uint64_t n, int nthreads, uint64_t grain, Fn fn) {
  if (nthreads < 1) nthreads = 1;
  uint64_t pieces = (n + grain - 1) / grain;
  if (pieces < (uint64_t)nthreads) nthreads = (int)std::max<uint64_t>(pieces, 1);
  if (nthreads <= 1) { fn(0, n); return; }
  std::vector<std::thread> th;
  uint64_t per = (n + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    uint64_t lo = std::min(n, (uint64_t)t * per), hi = std::min(n, lo + per);
    if (lo >= hi) break;
    th.emplace_back([=] { fn(lo, hi); });
  }
  for (auto& x : th) x.join();
}

inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  // inputs are finite N(0,1) variates; NaN handling is not needed here
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

// OCP 8-bit FP E4M3 ("fn": bias 7, no infinities, S.1111.111 = NaN), RNE with
// saturation to +-448.
uint8_t encode_e4m3(float v) {
  uint8_t sign = std::signbit(v) ? 0x80 : 0x00;
  double a = std::fabs((double)v);
  if (!(a < 448.0)) return sign | 0x7E;           // saturate (also catches inf)
  if (a < 0.015625) {                            // below 2^-6: subnormal step 2^-9
    double q = std::nearbyint(a * 512.0);        // 0..8; 8 is the min normal code
    return sign | (uint8_t)q;
  }
  int e;
  double m = std::frexp(a, &e);                  // a = m * 2^e, m in [0.5, 1)
  m *= 2.0;
  e -= 1;                                        // a = m * 2^e, m in [1, 2)
  double mq = std::nearbyint((m - 1.0) * 8.0);
  if (mq >= 8.0) { mq = 0.0; e += 1; }
  int ef = e + 7;
  if (ef > 15 || (ef == 15 && mq > 6.0)) return sign | 0x7E;
  return sign | (uint8_t)((ef << 3) | (int)mq);
}

// OCP E2M1 magnitude codes 0..7 are {0, .5, 1, 1.5, 2, 3, 4, 6}; RNE with
// saturation to 6.  Ties go to the code with an even mantissa bit.
uint8_t encode_e2m1(double v) {
  uint8_t sign = std::signbit(v) ? 0x8 : 0x0;
  double a = std::fabs(v);
  uint8_t c;
  if (a <= 0.25) c = 0;          // tie 0.25 -> 0 (even)
  else if (a < 0.75) c = 1;
  else if (a <= 1.25) c = 2;     // tie 0.75 -> 1.0 (code 2), tie 1.25 -> 1.0
  else if (a < 1.75) c = 3;
  else if (a <= 2.5) c = 4;      // tie 1.75 -> 2.0, tie 2.5 -> 2.0
  else if (a < 3.5) c = 5;
  else if (a <= 5.0) c = 6;      // tie 3.5 -> 4.0, tie 5.0 -> 4.0
  else c = 7;                    // saturate at 6
  return sign | c;
}

}  // namespace

extern "C" {

int kvgen_abi_version(void) { return 1; }

void kvgen_normal_f64(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count,
                      double* out, int nthreads) {
  uint64_t base = stream_base(seed, stream);
  parallel_for(count, nthreads, 1 << 16, [&](uint64_t lo, uint64_t hi) {
    normals_range(base, start + lo, hi - lo, [&](uint64_t k, double z) { out[lo + k] = z; });
  });
}

void kvgen_f32(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count, float* out,
               int nthreads) {
  uint64_t base = stream_base(seed, stream);
  parallel_for(count, nthreads, 1 << 16, [&](uint64_t lo, uint64_t hi) {
    normals_range(base, start + lo, hi - lo,
                  [&](uint64_t k, double z) { out[lo + k] = (float)z; });
  });
}

void kvgen_bf16(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count, uint16_t* out,
                int nthreads) {
  uint64_t base = stream_base(seed, stream);
  parallel_for(count, nthreads, 1 << 16, [&](uint64_t lo, uint64_t hi) {
    normals_range(base, start + lo, hi - lo,
                  [&](uint64_t k, double z) { out[lo + k] = f32_to_bf16_rne((float)z); });
  });
}

// fp8 E4M3 with one fp32 scale per slab.  Slab s (s = first_slab .. first_slab
// + nslabs - 1) is stream elements [s * slab_len, (s + 1) * slab_len).  Its
// scale is amax / 448 over the slab's fp32 values (1 if the slab is all zero),
// and each code is RNE(x / scale) in E4M3, saturated.  codes has nslabs *
// slab_len bytes, scales nslabs floats.
void kvgen_fp8_slabs(uint64_t seed, uint64_t stream, uint64_t first_slab, uint64_t nslabs,
                     uint64_t slab_len, uint8_t* codes, float* scales, int nthreads) {
  uint64_t base = stream_base(seed, stream);
  std::vector<float> buf(slab_len);
  int nt = nthreads < 1 ? 1 : nthreads;
  std::mutex mu;
  for (uint64_t s = 0; s < nslabs; ++s) {
    uint64_t e0 = (first_slab + s) * slab_len;
    float amax = 0.f;
    parallel_for(slab_len, nt, 1 << 16, [&](uint64_t lo, uint64_t hi) {
      float local = 0.f;
      normals_range(base, e0 + lo, hi - lo, [&](uint64_t k, double z) {
        float f = (float)z;
        buf[lo + k] = f;
        local = std::max(local, std::fabs(f));
      });
      std::lock_guard<std::mutex> g(mu);
      amax = std::max(amax, local);
    });
    float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    scales[s] = scale;
    uint8_t* dst = codes + s * slab_len;
    parallel_for(slab_len, nt, 1 << 16, [&](uint64_t lo, uint64_t hi) {
      for (uint64_t k = lo; k < hi; ++k) dst[k] = encode_e4m3(buf[k] / scale);
    });
  }
}

// OCP MXFP4: rows of D elements (D % 32 == 0) taken from stream elements
// [row * D, (row + 1) * D).  Each block of 32 contiguous elements gets an E8M0
// exponent E = clamp(floor(log2(amax)) - 2 + 127, 0, 254) (E = 127 for an
// all-zero block); elements are RNE(x / 2^(E-127)) in E2M1, saturated to +-6.
// data: nrows * D/2 bytes, element 2i in bits [3:0] of byte i and element
// 2i+1 in bits [7:4]; scales: nrows * D/32 bytes.
void kvgen_mxfp4(uint64_t seed, uint64_t stream, uint64_t start_row, uint64_t nrows, uint32_t D,
                 uint8_t* data, uint8_t* scales, int nthreads) {
  uint64_t base = stream_base(seed, stream);
  parallel_for(nrows, nthreads, 256, [&](uint64_t lo, uint64_t hi) {
    std::vector<float> row(D);
    for (uint64_t r = lo; r < hi; ++r) {
      normals_range(base, (start_row + r) * D, D,
                    [&](uint64_t k, double z) { row[k] = (float)z; });
      for (uint32_t blk = 0; blk < D / 32; ++blk) {
        const float* x = row.data() + blk * 32;
        float amax = 0.f;
        for (int k = 0; k < 32; ++k) amax = std::max(amax, std::fabs(x[k]));
        int E = 127;
        if (amax > 0.f) {
          int e2;
          std::frexp((double)amax, &e2);       // amax = m * 2^e2, m in [0.5, 1)
          int fl = e2 - 1;                     // floor(log2(amax))
          E = std::min(254, std::max(0, fl - 2 + 127));
        }
        scales[r * (D / 32) + blk] = (uint8_t)E;
        double inv = std::ldexp(1.0, -(E - 127));
        uint8_t* dst = data + r * (D / 2) + blk * 16;
        for (int k = 0; k < 16; ++k) {
          uint8_t lo4 = encode_e2m1((double)x[2 * k] * inv);
          uint8_t hi4 = encode_e2m1((double)x[2 * k + 1] * inv);
          dst[k] = (uint8_t)(lo4 | (hi4 << 4));
        }
      }
    }
  });
}

// Integers uniform in [lo, hi] (inclusive): lo + r(i) mod (hi - lo + 1).
void kvgen_uniform_int(uint64_t seed, uint64_t stream, uint64_t count, int64_t lo, int64_t hi,
                       int32_t* out) {
  uint64_t base = stream_base(seed, stream);
  uint64_t span = (uint64_t)(hi - lo) + 1;
  for (uint64_t i = 0; i < count; ++i) out[i] = (int32_t)(lo + (int64_t)(draw(base, i) % span));
}

// Encoders exposed for their own tests (values are encoded as the tensors
// above are).
void kvgen_encode_e4m3(const float* v, uint64_t n, uint8_t* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = encode_e4m3(v[i]);
}
void kvgen_encode_e2m1(const double* v, uint64_t n, uint8_t* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = encode_e2m1(v[i]);
}

}  // extern "C"
