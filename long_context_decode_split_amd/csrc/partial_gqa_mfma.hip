// Split-KV partial attention for a GQA group of 16 query heads on MFMA.
//
// With 16 query heads sharing one KV head, every cached K and V element feeds
// 16 multiply-adds, which is more arithmetic per HBM byte than the fp32 vector
// ALUs can sustain for fp8 or MXFP4 caches.  The 16 heads of the group are
// exactly the 16-wide dimension of the gfx950 matrix instructions, so both
// contractions run on them:
//
//   S^T[token, head] = K_tile[token, :] . Q[head, :]
//   O^T[dv, head]   += V_tile^T[dv, token] . P^T[token, head] (32 tokens, 8 column
//                                                              blocks x (hi, lo) = 16 MFMAs)
//
// The logits of a bf16 cache take four v_mfma_f32_16x16x32_bf16 per 16
// tokens.  An fp8 or MXFP4 K tile is not decoded at all: its bytes are the
// A operand of the block-scaled v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 with
// unit scales, or E2M1 with the cache's own E8M0 block exponents), and the
// bf16 query is the B operand as two E4M3 parts with power-of-two scales
// whose sum reproduces every query element that matters exactly (split_query),
// so the logits are exact products summed in fp32 in every format.  V is
// decoded to bf16 in registers with the hardware converters (exact).  The
// softmax weights P = exp2(logit - running max) are fp32; the PV product
// takes them as a bf16 pair hi + lo (two MFMAs), which keeps ~16 significant
// bits instead of 8, so the output error stays near fp32 level even for short
// shards.
//
// Work split: one workgroup of 4 waves per (shard j, request b, KV head,
// chunk of query tokens: one token for a single-token decode, two or four for
// a multi-token turn); wave w takes the shard's 32-token tiles w, w+4, w+8, ...
// and, for one token, keeps the loads of its next one (bf16) or two (fp8,
// MXFP4: smaller tiles) tiles in flight while computing the current one, so
// enough bytes are outstanding to cover HBM latency at 2-3 waves per SIMD.
// Several tokens share every loaded tile (see TW below).
// Lane (r, g) = (lane % 16, lane / 16):
//  * K: lane (r, g) loads token r of each 16-token half-tile, bytes
//    [64i + 16g, 64i + 16g + 16) of the row for each 16-byte load i, so each
//    load instruction reads 64 contiguous bytes of 16 rows.
//  * V: lane (r, g) loads columns [8r, 8r + 8) of the 8 tokens
//    {4g..4g+3, 16+4g..16+4g+3}, one full row per 16 lanes per instruction, and
//    regroups them with byte permutes into per-column token octets.
//  * The S^T output of the MFMA gives lane (n, g) head n at tokens
//    {4g+i, 16+4g+i}: exactly the P^T operand of the PV MFMA, so softmax state
//    (running max, partial sum) is per lane and needs no transposes; the O^T
//    accumulator of lane (n, g) is head n, dv in [32g, 32g + 32).
// The running max is only moved when a tile's max exceeds it by more than 2^8
// (in the exp2 domain); the stale max is exact algebra and keeps P <= 256.
// At the end the four waves' (max, sum, acc) states are merged through LDS and
// the normalized partial o and its natural-log lse are written.
#include <type_traits>

#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kD = 128;        // head width (Dqk = Dv)
constexpr int kTile = 32;      // tokens per wave iteration
constexpr float kLazyMax = 8.0f;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4_t v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  f32x2_t f = {x, y};
  bf16x2_t h = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Raw buffer resource (four SGPRs) over `bytes` bytes at a wave-uniform
// address.  Loads through it take a 32-bit lane offset plus an immediate, so a
// full tile needs no 64-bit per-lane address arithmetic; offsets at or past
// `bytes` would read zeros instead of memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, (int)bytes, 0x00020000);
}
template <bool NT>
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? 2 : 0));
}
template <bool NT>
__device__ __forceinline__ u32x2_t buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, NT ? 2 : 0));
}
template <bool NT>
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, NT ? 2 : 0);
}
template <bool NT>
__device__ __forceinline__ uint32_t buf_load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, NT ? 2 : 0);
}

template <int KV>
struct Layout;

// bf16: 64 B of K per lane per half-tile (4 loads), 16 B of V per token.
template <>
struct Layout<kBF16> {
  static constexpr int kRing = 2;       // tiles held in registers (current + prefetched)
  static constexpr int kKLoads = 4;     // 16-byte K loads per lane per half-tile
  static constexpr int kVBytes = 16;    // V bytes per lane per token
  static constexpr int kRowBytes = 256;
  // first d of MFMA chunk c for lane group g
  __device__ static constexpr int chunk_d(int c, int g) { return 32 * c + 8 * g; }
};
// kFmt: the A operand format code of the block-scaled MFMA (cbsz).
template <>
struct Layout<kFP8> {
  static constexpr int kFmt = 0;        // E4M3; lane (r, g) holds dims 16g.. and 64+16g..
  static constexpr int kRing = 3;
  static constexpr int kKLoads = 2;
  static constexpr int kVBytes = 8;
  static constexpr int kRowBytes = 128;
};
template <>
struct Layout<kMXFP4> {
  static constexpr int kFmt = 4;        // E2M1; lane (r, g) holds dims 32g .. 32g+31
  static constexpr int kRing = 3;
  static constexpr int kKLoads = 1;
  static constexpr int kVBytes = 4;
  static constexpr int kRowBytes = 64;
};

// Raw (undecoded) registers of one 32-token tile for one lane.
template <int KV>
struct Raw {
  uint32_t k[2][Layout<KV>::kKLoads * 4];      // two half-tiles
  uint32_t v[8][Layout<KV>::kVBytes / 4];      // 8 tokens
  uint32_t ks[2];                              // MXFP4: K block exponent per half-tile
  uint32_t vs[2];                              // MXFP4: byte `lane` of the half-tile's V exponents
};

// LDS ring of the multi-token kernel (bf16 cache): per wave, kSlots raw
// tiles filled by direct-to-LDS loads.  A tile is 32 rows of K then 32 rows
// of V, each half of 16 rows a contiguous copy of 16 cache rows.
struct Ring {
  static constexpr int kRow = Layout<kBF16>::kRowBytes;
  static constexpr int kSlots = 2;
  static constexpr int kTileBytes = 2 * kTile * kRow;
  static constexpr int kDmaPerHalf = 16 * kRow / 1024;   // 1 KB per load instruction
  static constexpr int kDmaPerTile = 4 * kDmaPerHalf;
  static constexpr int kWaveBytes = kSlots * kTileBytes;
};

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

// Longest-request-first order of the shard units.  Position p of the unit
// queue (workgroups start roughly in id order) takes a unit of the request
// ranked p / (kvp Hkv) by sequence length, longest first (ties by index), so
// the longest shards start first and the short ones fill the tail of the
// grid.  Lane b of the wave holds request b's length and counts the requests
// ahead of it; up to 64 requests.  Larger batches, and batches whose requests
// all have one length, keep the plain (shard-major) order.  Every unit keeps
// its (shard, KV head) and every request keeps its units, so this only
// permutes which workgroup does which unit.
__device__ __forceinline__ int64_t longest_first_unit(int64_t p, const PartialArgs& a) {
  if (a.B <= 1 || a.B > 64) return p;
  const int per = a.kvp * a.Hkv;
  const int r = (int)(p / per);
  const int rem = (int)(p - (int64_t)r * per);
  const int lane = threadIdx.x & 63;
  const int my = lane < a.B ? a.seq_lens[lane] : -1;
  if (__ballot(lane < a.B && my != __builtin_amdgcn_readfirstlane(my)) == 0) return p;
  int ahead = 0;
  for (int b2 = 0; b2 < a.B; ++b2) {
    const int o = __builtin_amdgcn_readlane(my, b2);
    ahead += (o > my || (o == my && b2 < lane)) ? 1 : 0;
  }
  const uint64_t hit = __ballot(lane < a.B && ahead == r);
  const int b = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
  return ((int64_t)(rem / a.Hkv) * a.B + b) * a.Hkv + rem % a.Hkv;
}

// LDS of the final merge of the four waves' states.
struct MergeLds {
  float o[kWaves][16][kD + 4];
  float m[kWaves][16];
  float l[kWaves][16];
};

// bf16 K operand of MFMA chunk c of half-tile u: the 8 dims
// Layout<kBF16>::chunk_d(c, g) of token 16u + r16.
__device__ __forceinline__ bf16x8_t k_operand(const Raw<kBF16>& rw, int u, int c) {
  return as_bf16x8(rw.k[u][4 * c], rw.k[u][4 * c + 1], rw.k[u][4 * c + 2], rw.k[u][4 * c + 3]);
}

// The K bytes of half-tile u as the A operand of the block-scaled MFMA: an
// fp8 lane holds 32 E4M3 bytes, an MXFP4 lane 16 bytes (32 E2M1 nibbles, the
// upper half of the operand unused).
template <int KV>
__device__ __forceinline__ i32x8_t k_bytes(const Raw<KV>& rw, int u) {
  i32x8_t a;
#pragma unroll
  for (int w = 0; w < 8; ++w) a[w] = w < 4 * Layout<KV>::kKLoads ? (int)rw.k[u][w] : 0;
  return a;
}

// The query of head n as the B operand of v_mfma_scale_f32_16x16x128_f8f6f4
// (fp8 and MXFP4 caches).  With 8-bit operands lane group g of that
// instruction covers the contraction indices {16g .. 16g+15, 64+16g .. 64+16g+15}
// (bytes 0-15, 16-31) and supplies the E8M0 scale of index block g
// (32g .. 32g+31); with a 4-bit A operand lane group g covers 32g .. 32g+31.
// One scale per head, so the per-lane scales agree whatever the grouping.
// The bf16 query is split as q = hi 2^sh + lo 2^sl, hi and lo OCP E4M3 and
// round-to-nearest: sh puts the head's largest |q| in [128, 256) hi units and
// sl = sh - 4.  Where |q| >= 2^(sh-6) (hi normal), the residual q - hi 2^sh is
// a multiple of q's ulp of at most half an E4M3 ulp of q, so it has at most
// 4 significant bits and lo holds it exactly: hi 2^sh + lo 2^sl = q.  Smaller
// elements (below 2^-13 of the head's largest |q|) are off by at most half an
// E4M3 subnormal step of lo, 2^(sl-10) = 2^(sh-14).
struct QSplit {
  i32x8_t hi, lo;
  int sh, sl;   // E8M0 scale bytes (exponent + 127)
};

__device__ __forceinline__ QSplit split_query(const uint16_t* qrow, int g) {
  float x[32];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint4 v = *reinterpret_cast<const uint4*>(qrow + 64 * h + 16 * g + 8 * k);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[16 * h + 8 * k + 2 * e] = __uint_as_float(w[e] << 16);
        x[16 * h + 8 * k + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = rows4_max(amax);   // the head's 128 dims sit in its 4 lane groups
  // floor(log2(amax)) from the exponent field (amax = 0 or fp32-subnormal: the
  // clamp below takes over)
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 127;
  int sh = e - 7;
  sh = sh < -123 ? -123 : (sh > 120 ? 120 : sh);
  const int sl = sh - 4;
  const float inv_h = __uint_as_float((uint32_t)(127 - sh) << 23);   // 2^-sh, exact
  QSplit r;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    float y[4], z[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] = x[4 * w + k] * inv_h;
    int hw = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    hw = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], hw, true);
    const f32x2_t h01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)hw, 1.0f, false);
    const f32x2_t h23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)hw, 1.0f, true);
    // residual in lo units (exact: y - hi is on y's grid, 16 a power of two)
    z[0] = (y[0] - h01[0]) * 16.0f;
    z[1] = (y[1] - h01[1]) * 16.0f;
    z[2] = (y[2] - h23[0]) * 16.0f;
    z[3] = (y[3] - h23[1]) * 16.0f;
    int lw = __builtin_amdgcn_cvt_pk_fp8_f32(z[0], z[1], 0, false);
    lw = __builtin_amdgcn_cvt_pk_fp8_f32(z[2], z[3], lw, true);
    r.hi[w] = hw;
    r.lo[w] = lw;
  }
  r.sh = sh + 127;
  r.sl = sl + 127;
  return r;
}

// V^T operands of the 8 16-column blocks of the PV product, decoded to bf16:
// f(blk, op) is called for each block as soon as its operand is ready.  The
// operand of block blk holds the lane's column of that block for the 8 tokens
// {4g + i, 16 + 4g + i}, in the k order of the P^T operand.
// MXFP4: lane L of the wave holds the V exponent of (token 16u + L / 4,
// column block L % 4) in rw.vs[u]; vs_lane is the byte address (for
// ds_bpermute) of the lane holding this lane's block (r / 4) of token 4g.
template <int KV, class F>
__device__ __forceinline__ void for_v_operands(const Raw<KV>& rw, uint32_t vs_lane, F&& f) {
  if constexpr (KV == kBF16 || KV == kMXFP4) {
    // token-major bf16 pairs cv[e][q] = columns (8 r16 + 2q, 8 r16 + 2q + 1) of token e
    uint32_t cv[8][4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (KV == kBF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) cv[e][q] = rw.v[e][q];
      } else {
        // token 16 (e / 4) + 4g + e % 4 sits 4 (e % 4) lanes past token 4g
        const uint32_t x = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(vs_lane + 16 * (e % 4)), (int)rw.vs[e / 4]);
        const float vsc = e8m0_to_f32_fast(x);
        const uint32_t w = rw.v[e][0];
        cv[e][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, vsc, 0));
        cv[e][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, vsc, 1));
        cv[e][2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, vsc, 2));
        cv[e][3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, vsc, 3));
      }
    }
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const int q = blk / 2;
      const uint32_t sel = (blk & 1) ? 0x07060302u : 0x05040100u;
      f(blk, as_bf16x8(perm(cv[1][q], cv[0][q], sel), perm(cv[3][q], cv[2][q], sel),
                       perm(cv[5][q], cv[4][q], sel), perm(cv[7][q], cv[6][q], sel)));
    }
  } else {
    // fp8: interleave bytes of token pairs, then convert both halves
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int s2 = 0; s2 < 4; s2 += 2) {
        const uint32_t sel = (s2 == 0) ? 0x05010400u : 0x07030602u;
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const uint32_t x2 = perm(rw.v[2 * rr + 1][q], rw.v[2 * rr][q], sel);
          lo[rr] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x2, 1.0f, false));
          hi[rr] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x2, 1.0f, true));
        }
        f(4 * q + s2, as_bf16x8(lo[0], lo[1], lo[2], lo[3]));
        f(4 * q + s2 + 1, as_bf16x8(hi[0], hi[1], hi[2], hi[3]));
      }
    }
  }
}

// PAGED: rows are found through the block table (paged cache layout).
// NT: cache loads carry the non-temporal hint: every cache byte is read once
// when one token chunk covers all query tokens.  With several chunks each
// chunk reads the shard's rows, the loads are plain, and the later chunks of
// a shard find them in the caches.
// TW: query tokens per workgroup.  Each wave loads a tile (and decodes its V)
// once and runs the logits, softmax and PV product of each of the TW tokens on
// it; every token keeps its own Q operands, softmax state and accumulator.
// LDSRING: the tiles ahead wait in an LDS ring filled by direct-to-LDS loads
// (Ring, bf16 cache) instead of in registers, which leaves the registers to the
// tokens and keeps several tiles in flight at one wave per SIMD.
template <int KV, bool PAGED, bool NT, int TW, bool LDSRING>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(KV != kBF16 && TW == 1 ? 3 : 1)))
void gqa_mfma_kernel(PartialArgs a) {
  using Lay = Layout<KV>;
  constexpr int64_t ROW = Lay::kRowBytes;
  constexpr int kRing = TW > 1 ? 2 : Lay::kRing;

  MergeLds* mrg;
  uint32_t ring_lds = 0;   // LDSRING: LDS address of this wave's slots
  if constexpr (LDSRING) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
    mrg = reinterpret_cast<MergeLds*>(dyn_lds);   // reused once the ring is drained
    ring_lds = (uint32_t)(uintptr_t)(lds_u8*)dyn_lds +
               (uint32_t)(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * Ring::kWaveBytes);
  } else {
    __shared__ MergeLds st;
    mrg = &st;
  }

  const int lane = threadIdx.x & 63;
  // wave index as a scalar, so everything derived from it stays wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;

  // unit (shard j, request b, KV head kvh) and chunk of TW query tokens
  const int nchunks = (a.T + TW - 1) / TW;
  int64_t unit;
  int chunk;
  if (!unit_token(blockIdx.x, (int64_t)a.kvp * a.B * a.Hkv, nchunks, &unit, &chunk)) return;
  unit = longest_first_unit(unit, a);
  const int kvh = (int)(unit % a.Hkv);
  const int b = (int)(unit / a.Hkv % a.B);
  const int j = (int)(unit / ((int64_t)a.Hkv * a.B));
  const int qt0 = chunk * TW;                       // first query token of the chunk
  const int nq = a.T - qt0 < TW ? a.T - qt0 : TW;   // tokens of the chunk that exist

  // The rows the shard holds are [s0, s1); token i of the chunk sees rows
  // [s0, s1t[i]) (its causal cut).  Later tokens see more, so the last one
  // bounds the rows read; tokens past the end of T see none.
  const int64_t L = a.seq_lens[b];
  const ShardSpan span = shard_span(a.layout, L, a.T, qt0 + nq - 1, a.S_max, a.kvp, a.B, a.Hkv, j, b, kvh);
  const int64_t s0 = span.s0, s1 = span.s1;
  int64_t s1t[TW];
#pragma unroll
  for (int i = 0; i < TW; ++i)
    s1t[i] = i >= nq ? s0 : (i == nq - 1 ? s1 : shard_span(a.layout, L, a.T, qt0 + i, a.S_max, a.kvp, a.B, a.Hkv,
                                                            j, b, kvh).s1);
  const int64_t slab = span.slab;                  // cache block of this shard
  const int64_t bh = (int64_t)b * a.Hkv + kvh;     // fp8 scales are per (request, KV head)
  const int ntiles = (int)((s1 - s0 + kTile - 1) / kTile);

  // The cache arrays are viewed as rows of ROW bytes (scales: kD/32 bytes).
  // Contiguous and sharded layouts: token t of this shard is row
  // slab * S_max + t, so pointers start at the slab; paged: rows come from
  // the block table (phys_row) and pointers start at the pool.
  const int64_t row0 = PAGED ? 0 : slab * a.S_max;
  const uint8_t* kdata = static_cast<const uint8_t*>(a.k) + row0 * ROW;
  const uint8_t* vdata = static_cast<const uint8_t*>(a.v) + row0 * ROW;
  const uint8_t* ksdata = nullptr;
  const uint8_t* vsdata = nullptr;
  auto hrow = [&](int64_t t) -> int64_t {
    if constexpr (PAGED) {
      return phys_row(a, b, kvh, slab, t);
    } else {
      return t;
    }
  };
  float kscale = 1.0f, vscale = 1.0f;
  if constexpr (KV == kFP8) {
    kscale = static_cast<const float*>(a.k_scale)[bh];
    vscale = static_cast<const float*>(a.v_scale)[bh];
  }
  if constexpr (KV == kMXFP4) {
    ksdata = static_cast<const uint8_t*>(a.k_scale) + row0 * (kD / 32);
    vsdata = static_cast<const uint8_t*>(a.v_scale) + row0 * (kD / 32);
  }
  const float c2 = a.scale_log2 * kscale;  // raw logit -> log2 domain

  // Q^T operands of each token of the chunk (a token past the end of T loads
  // the last one's): bf16 cache, lane (n, g) holds head n, the 8 d of chunk c
  // for group g; fp8 and MXFP4 caches, the two E4M3 parts of split_query.
  constexpr bool SCALED = KV != kBF16;
  bf16x8_t qop[TW][4];
  QSplit qs[TW];
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    const int qt = qt0 + (i < nq ? i : nq - 1);
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (((int64_t)b * a.T + qt) * a.Hq + kvh * 16 + r16) * kD;
    if constexpr (SCALED) {
      qs[i] = split_query(qrow, g);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 v = *reinterpret_cast<const uint4*>(qrow + Lay::chunk_d(c, g));
        qop[i][c] = as_bf16x8(v.x, v.y, v.z, v.w);
      }
    }
  }

  f32x4_t acc[TW][8];
  float m2[TW];    // running max of this lane's head (log2 domain)
  float lsum[TW];  // partial sum of P over this lane's tokens
#pragma unroll
  for (int i = 0; i < TW; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[i][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m2[i] = -INFINITY;
    lsum[i] = 0.0f;
  }

  const int64_t last = s1 - 1;
  // Per-lane byte offsets inside a tile (loop invariant, 32-bit): a full tile
  // is addressed as (wave-uniform tile pointer) + (lane offset) + (immediate),
  // which needs no per-load vector arithmetic.
  const uint32_t koff = (uint32_t)(r16 * ROW + 16 * g);
  const uint32_t voff = (uint32_t)(4 * g * ROW + Lay::kVBytes * r16);
  const uint32_t ksoff = (uint32_t)(r16 * (kD / 32) + g);
  // MXFP4 V scales: the 64 exponent bytes of a half-tile (16 tokens x 4
  // column blocks) are one byte per lane, lane L holding byte L; the lane that
  // holds this lane's block r16 / 4 of token 4g is 16g + r16 / 4.
  const uint32_t vs_lane = (uint32_t)(4 * (16 * g + r16 / 4));

  // FULL: every row of the tile is inside the shard (no clamping needed).
  // Each 16-token half-tile is 16 consecutive physical rows starting at
  // hr[u]; rows of a partial tile are clamped to the shard's last token.
  constexpr int64_t SROW = kD / 32;   // MXFP4 scale bytes per row
  auto load = [&](Raw<KV>& rw, int tile, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int64_t base = s0 + (int64_t)tile * kTile;
    if constexpr (FULL) {
      // every load of a half-tile through one buffer resource over its 16 rows
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t hr = hrow(base + 16 * u);
        const auto rk = tile_rsrc(kdata + hr * ROW, 16 * ROW);
#pragma unroll
        for (int i = 0; i < Lay::kKLoads; ++i) {
          const u32x4_t v = buf_load16<NT>(rk, koff + 64 * i);
#pragma unroll
          for (int w = 0; w < 4; ++w) rw.k[u][4 * i + w] = v[w];
        }
        const auto rv = tile_rsrc(vdata + hr * ROW, 16 * ROW);
#pragma unroll
        for (int e = 4 * u; e < 4 * u + 4; ++e) {   // token 16u + 4g + e%4
          const uint32_t off = voff + (uint32_t)((e % 4) * ROW);
          if constexpr (Lay::kVBytes == 16) {
            const u32x4_t v = buf_load16<NT>(rv, off);
#pragma unroll
            for (int w = 0; w < 4; ++w) rw.v[e][w] = v[w];
          } else if constexpr (Lay::kVBytes == 8) {
            const u32x2_t v = buf_load8<NT>(rv, off);
            rw.v[e][0] = v[0];
            rw.v[e][1] = v[1];
          } else {
            rw.v[e][0] = buf_load4<NT>(rv, off);
          }
        }
        if constexpr (KV == kMXFP4) {
          rw.ks[u] = buf_load1<NT>(tile_rsrc(ksdata + hr * SROW, 16 * SROW), ksoff);
          rw.vs[u] = buf_load1<NT>(tile_rsrc(vsdata + hr * SROW, 16 * SROW), (uint32_t)lane);
        }
      }
    } else {
      // partial tile: rows past the shard's last one are clamped, lane by lane
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        int64_t t = base + 16 * u + r16;
        t = t < last ? t : last;
        const int64_t pt = hrow(t);
        const uint8_t* p = kdata + pt * ROW + 16 * g;
#pragma unroll
        for (int i = 0; i < Lay::kKLoads; ++i) {
          const u32x4_t v = stream_load16<NT>(p + 64 * i);
#pragma unroll
          for (int w = 0; w < 4; ++w) rw.k[u][4 * i + w] = v[w];
        }
        if constexpr (KV == kMXFP4) {
          rw.ks[u] = stream_load1<NT>(ksdata + pt * SROW + g);
          int64_t tv = base + 16 * u + lane / 4;
          tv = tv < last ? tv : last;
          rw.vs[u] = stream_load1<NT>(vsdata + hrow(tv) * SROW + (lane & 3));
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int64_t t = base + 16 * (e / 4) + (e % 4) + 4 * g;
        t = t < last ? t : last;
        const uint8_t* p = vdata + hrow(t) * ROW + Lay::kVBytes * r16;
        if constexpr (Lay::kVBytes == 16) {
          const u32x4_t v = stream_load16<NT>(p);
#pragma unroll
          for (int w = 0; w < 4; ++w) rw.v[e][w] = v[w];
        } else if constexpr (Lay::kVBytes == 8) {
          const u32x2_t v = stream_load8<NT>(p);
          rw.v[e][0] = v[0];
          rw.v[e][1] = v[1];
        } else {
          rw.v[e][0] = stream_load4<NT>(p);
        }
      }
    }
  };

  // Logits S^T = K Q^T of query token i of the chunk for the two half-tiles,
  // as 8 values per lane: head n = r16, tokens base + 16u + 4g + i at x[4u + i].
  // bf16: kop holds the K operands (filled here for one token); fp8 and
  // MXFP4: two block-scaled MFMAs per half-tile (query parts hi and lo) on the
  // raw K bytes.
  auto logits = [&](const Raw<KV>& rw, bf16x8_t (&kop)[2][4], int i, float (&x)[8]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (SCALED) {
        const i32x8_t ka = k_bytes<KV>(rw, u);
        const int ksc = KV == kMXFP4 ? (int)rw.ks[u] : 127;   // E8M0 1.0 for fp8
        s = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qs[i].hi, s, Lay::kFmt, 0, 0, ksc, 0, qs[i].sh);
        s = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qs[i].lo, s, Lay::kFmt, 0, 0, ksc, 0, qs[i].sl);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if constexpr (TW == 1) kop[u][c] = k_operand(rw, u, c);
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[u][c], qop[i][c], s, 0, 0, 0);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * u + e] = s[e];
    }
  };
  // Max of the lane's 8 logits of its head, in the log2 domain.  Whether the
  // running max must move is decided on these lane maxima (any lane over its
  // head's max + 2^kLazyMax); only then is the head's tile max reduced over
  // its 4 lane groups, so all 4 keep the same running max.
  auto lane_max2 = [&](const float (&x)[8]) {
    float tmax = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, x[e]);
    return tmax * c2;
  };
  // Move the running max to mn, rescaling the state.
  auto rescale = [&](float& m, float& l, f32x4_t (&o)[8], float mn) {
    const float al = fast_exp2(m - mn);
    l *= al;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= al;
    m = mn;
  };
  // Softmax weights P = 2^(x c2 - m) (0 for masked logits) added to the
  // running sum and split as P = hi + lo: hi keeps the upper 16 bits of each
  // fp32 weight (exact), lo is the remainder rounded to bf16, so hi + lo
  // carries ~16 significant bits.
  auto weights = [&](const float (&x)[8], float m, float& l, bf16x8_t& pop, bf16x8_t& pol, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = fast_exp2(fmaf(x[e], c2, -m));
      if constexpr (MASK) p[e] = (x[e] == -INFINITY) ? 0.0f : p[e];
      l += p[e];
    }
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const uint32_t b0 = __float_as_uint(p[2 * rr]), b1 = __float_as_uint(p[2 * rr + 1]);
      ph[rr] = perm(b1, b0, 0x07060302u);
      pl[rr] = pack_bf16(p[2 * rr] - __uint_as_float(b0 & 0xFFFF0000u),
                         p[2 * rr + 1] - __uint_as_float(b1 & 0xFFFF0000u));
    }
    pop = as_bf16x8(ph[0], ph[1], ph[2], ph[3]);
    pol = as_bf16x8(pl[0], pl[1], pl[2], pl[3]);
  };

  // One query token on one tile: logits, the online softmax update of head
  // n = r16 over tokens base + 16u + 4g + i, and O^T += V^T P^T, each K and V
  // operand decoded next to its use.  MASK: rows from nvalid on are not seen
  // (zero weight).  The running max only moves when a tile's max exceeds it
  // by more than 2^kLazyMax (in the exp2 domain).
  auto token_tile = [&](const Raw<KV>& rw, bf16x8_t (&kop)[2][4], float& m, float& l, f32x4_t (&o)[8], int nvalid,
                        auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    float x[8];
    logits(rw, kop, 0, x);
    if constexpr (MASK) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * u + 4 * g + i >= nvalid) x[4 * u + i] = -INFINITY;
    }
    const float lmax2 = lane_max2(x);
    if (__any(lmax2 > m + kLazyMax)) rescale(m, l, o, fmaxf(m, rows4_max(lmax2)));
    bf16x8_t pop, pol;
    weights(x, m, l, pop, pol, mask_tag);
    // one MFMA pair per 16-column block
    auto pv = [&](int blk, const bf16x8_t& v) {
      o[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, pop, o[blk], 0, 0, 0);
      o[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, pol, o[blk], 0, 0, 0);
    };
    for_v_operands<KV>(rw, vs_lane, pv);
  };

  // Every token of the chunk on one tile, phase by phase: the K operands (bf16:
  // repacked once; fp8, MXFP4: the raw bytes) for the logits of all tokens, one
  // rescale check, the weights of all, then V
  // decoded block by block straight into every token's PV product.  The
  // tokens' independent MFMA chains interleave, and neither all K nor all V
  // operands are held at once.  MASK: token i sees the tile's rows below
  // nv[i] only (none when nv[i] <= 0).
  auto tokens_tile = [&](const Raw<KV>& rw, const int (&nv)[TW], auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    float x[TW][8];
    {
      bf16x8_t kop[2][4];
      if constexpr (!SCALED) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int c = 0; c < 4; ++c) kop[u][c] = k_operand(rw, u, c);
      }
#pragma unroll
      for (int i = 0; i < TW; ++i) logits(rw, kop, i, x[i]);
    }
    if constexpr (MASK) {
#pragma unroll
      for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (16 * u + 4 * g + e >= nv[i]) x[i][4 * u + e] = -INFINITY;
    }
    float lmax2[TW];
    bool need = false;
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      lmax2[i] = lane_max2(x[i]);
      need = need || (lmax2[i] > m2[i] + kLazyMax);
    }
    if (__any(need)) {
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        const float tmax2 = rows4_max(lmax2[i]);
        if (__any(tmax2 > m2[i] + kLazyMax)) rescale(m2[i], lsum[i], acc[i], fmaxf(m2[i], tmax2));
      }
    }
    bf16x8_t pop[TW], pol[TW];
#pragma unroll
    for (int i = 0; i < TW; ++i) weights(x[i], m2[i], lsum[i], pop[i], pol[i], mask_tag);
    for_v_operands<KV>(rw, vs_lane, [&](int blk, const bf16x8_t& v) {
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        acc[i][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, pop[i], acc[i][blk], 0, 0, 0);
        acc[i][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, pol[i], acc[i][blk], 0, 0, 0);
      }
    });
  };

  // MASK: the tile runs past the shard end (single token: its extra tokens get
  // zero weight).  With several tokens every token checks its own cut.
  using Masked = std::true_type;      // compute: rows past a token's cut get weight 0
  using Unmasked = std::false_type;
  using FullTile = std::true_type;    // load: every row of the tile inside the shard
  using PartTile = std::false_type;
  using Clamped = std::true_type;     // issue: rows clamped to the shard, lane by lane
  using Unclamped = std::false_type;
  auto compute = [&](const Raw<KV>& rw, int tile, auto mask_tag) {
    const int64_t base = s0 + (int64_t)tile * kTile;
    if constexpr (TW == 1) {
      bf16x8_t kop[2][4];
      token_tile(rw, kop, m2[0], lsum[0], acc[0], (int)(s1 - base), mask_tag);
    } else {
      int nv[TW];
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        const int64_t n = s1t[i] - base;         // wave-uniform
        nv[i] = n < 0 ? 0 : (n > kTile ? kTile : (int)n);
      }
      if (nv[0] == kTile)                        // every token sees the whole tile
        tokens_tile(rw, nv, Unmasked{});
      else
        tokens_tile(rw, nv, Masked{});
    }
  };

  const int nfull = (int)((s1 - s0) / kTile);
  if constexpr (LDSRING) {
    static_assert(KV == kBF16, "LDS ring: bf16 cache only");
    using R = Ring;
    // Direct-to-LDS loads of tile `tile` into slot sl.  Full tile: each half
    // is 16 consecutive rows, copied 1 KB per instruction from a wave-uniform
    // base.  Partial tile (CLAMP): rows past the shard's last one are clamped,
    // lane by lane.
    auto issue = [&](int tile, int sl, auto clamp_tag) {
      constexpr bool CLAMP = decltype(clamp_tag)::value;
      const int64_t base = s0 + (int64_t)tile * kTile;
      const uint32_t dst = ring_lds + (uint32_t)(sl * R::kTileBytes);
      int64_t hr[2] = {0, 0};
      if constexpr (!CLAMP) {
        hr[0] = hrow(base);
        hr[1] = hrow(base + 16);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int n = 0; n < R::kDmaPerHalf; ++n) {
          const uint32_t off = (uint32_t)(n * 1024 + 16 * lane);   // byte of the half-tile
          const uint32_t m0k = __builtin_amdgcn_readfirstlane(dst + (uint32_t)(u * 16 * ROW + n * 1024));
          const uint32_t m0v = m0k + (uint32_t)(kTile * ROW);
          if constexpr (CLAMP) {
            int64_t t = base + 16 * u + off / ROW;
            t = t < last ? t : last;
            const int64_t pr = hrow(t) * ROW + off % ROW;
            lds_dma16_at(m0k, kdata + pr);
            lds_dma16_at(m0v, vdata + pr);
          } else {
            lds_dma16<NT>(m0k, kdata + hr[u] * ROW, off);
            lds_dma16<NT>(m0v, vdata + hr[u] * ROW, off);
          }
        }
      }
    };
    // The raw registers of slot sl, in the lane layout of the register loads.
    auto fetch = [&](Raw<KV>& rw, int sl) {
      const lds_u8* sp = (const lds_u8*)(uintptr_t)(ring_lds + (uint32_t)(sl * R::kTileBytes));
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int i = 0; i < Lay::kKLoads; ++i) {
          const u32x4_t v = *(const lds_u32x4*)(sp + u * 16 * ROW + koff + 64 * i);
#pragma unroll
          for (int w = 0; w < 4; ++w) rw.k[u][4 * i + w] = v[w];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const lds_u8* p = sp + kTile * ROW + (16 * (e / 4) + (e % 4)) * ROW + voff;
        if constexpr (Lay::kVBytes == 16) {
          const u32x4_t v = *(const lds_u32x4*)p;
#pragma unroll
          for (int w = 0; w < 4; ++w) rw.v[e][w] = v[w];
        } else if constexpr (Lay::kVBytes == 8) {
          const u32x2_t v = *(const lds_u32x2*)p;
          rw.v[e][0] = v[0];
          rw.v[e][1] = v[1];
        } else {
          rw.v[e][0] = *(const lds_u32*)p;
        }
      }
    };
    // Every vector memory operation in flight from here on is a ring load.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    if (nfull > 0) {
      auto clampt = [&](int t) { return t < nfull - 1 ? t : nfull - 1; };
#pragma unroll
      for (int k = 0; k < R::kSlots - 1; ++k) issue(clampt(wave + k * kWaves), k, Unclamped{});
      int sl = 0;
      for (int tile = wave; tile < nfull; tile += kWaves) {
        // refill the slot read in the previous iteration, kSlots - 1 tiles ahead
        issue(clampt(tile + (R::kSlots - 1) * kWaves), sl == 0 ? R::kSlots - 1 : sl - 1, Unclamped{});
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((R::kSlots - 1) * R::kDmaPerTile));
        asm volatile("" ::: "memory");
        Raw<KV> rw;
        fetch(rw, sl);
        compute(rw, tile, Unmasked{});
        sl = sl + 1 == R::kSlots ? 0 : sl + 1;
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      asm volatile("" ::: "memory");
    }
    if (nfull < ntiles && nfull % kWaves == wave) {
      issue(nfull, 0, Clamped{});
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      asm volatile("" ::: "memory");
      Raw<KV> rt;
      fetch(rt, 0);
      compute(rt, nfull, Masked{});
    }
    __syncthreads();   // every wave is done with its slots before the merge reuses them
  } else {
    // Stream over this wave's full tiles with kRing register buffers: the loads
    // of the next kRing-1 tiles are in flight while a tile is computed.  (With
    // several query tokens a tile takes several times longer to compute, so
    // one tile ahead is enough and leaves the registers to the tokens.)  The
    // next loads are always issued (clamped to the last full tile) so the waits
    // stay static.  A partial last tile is handled once, after the ring.
    if (nfull > 0) {
      auto clampt = [&](int t) { return t < nfull - 1 ? t : nfull - 1; };
      int tile = wave;
      if constexpr (kRing == 2) {
        Raw<KV> ra, rb;
        load(ra, clampt(tile), FullTile{});
        while (tile < nfull) {
          load(rb, clampt(tile + kWaves), FullTile{});
          compute(ra, tile, Unmasked{});
          tile += kWaves;
          if (tile >= nfull) break;
          load(ra, clampt(tile + kWaves), FullTile{});
          compute(rb, tile, Unmasked{});
          tile += kWaves;
        }
      } else {
        static_assert(kRing == 3, "ring of 2 or 3 buffers");
        Raw<KV> ra, rb, rc;
        load(ra, clampt(tile), FullTile{});
        load(rb, clampt(tile + kWaves), FullTile{});
        while (tile < nfull) {
          load(rc, clampt(tile + 2 * kWaves), FullTile{});
          compute(ra, tile, Unmasked{});
          tile += kWaves;
          if (tile >= nfull) break;
          load(ra, clampt(tile + 2 * kWaves), FullTile{});
          compute(rb, tile, Unmasked{});
          tile += kWaves;
          if (tile >= nfull) break;
          load(rb, clampt(tile + 2 * kWaves), FullTile{});
          compute(rc, tile, Unmasked{});
          tile += kWaves;
        }
      }
    }
    if (nfull < ntiles && nfull % kWaves == wave) {
      Raw<KV> rt;
      load(rt, nfull, PartTile{});
      compute(rt, nfull, Masked{});
    }
  }
  // ---- merge the four waves' states of each token and write its partial
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    if (i >= nq) break;
    const float lw = rows4_sum(lsum[i]);
    if (i > 0) __syncthreads();        // the previous token's reads are done
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) mrg->o[wave][r16][32 * g + 8 * e + blk] = acc[i][blk][e];
    }
    if (g == 0) {
      mrg->m[wave][r16] = m2[i];
      mrg->l[wave][r16] = lw;
    }
    __syncthreads();
    const int64_t orow0 = (((int64_t)j * a.B + b) * a.T + qt0 + i) * a.Hq + kvh * 16;   // o_part / lse_part row
    const int tid = threadIdx.x;
    for (int idx = tid; idx < 16 * kD; idx += kThreads) {
      const int n = idx / kD;
      const int d = idx - n * kD;
      float M = mrg->m[0][n];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mrg->m[w][n]);
      float o = 0.0f;
      if (M != -INFINITY) {
        float lt = 0.0f, ot = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float f = rescale_weight(mrg->m[w][n], M);
          lt += mrg->l[w][n] * f;
          ot += mrg->o[w][n][d] * f;
        }
        o = ot / lt * vscale;
      }
      a.o_part[(orow0 + n) * kD + d] = o;
    }
    if (tid < 16) {
      float M = mrg->m[0][tid];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mrg->m[w][tid]);
      float lse = -INFINITY;
      if (M != -INFINITY) {
        float lt = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) lt += mrg->l[w][tid] * rescale_weight(mrg->m[w][tid], M);
        lse = (M + fast_log2(lt)) * kLn2;
      }
      a.lse_part[orow0 + tid] = lse;
    }
  }
}

}  // namespace

bool gqa_mfma_supports(const PartialArgs& a) {
  if (!a.q_bf16 || a.v_aliases_k) return false;
  if (a.Dqk != kD || a.Dv != kD) return false;
  if (a.Hq / a.Hkv != 16) return false;
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

// The four-token instance (bf16 cache, LDS ring of tiles) with NT loads or not.
template <int KV, bool PAGED, bool NT>
hipError_t launch_gqa_ring(const PartialArgs& a, dim3 grid, hipStream_t stream) {
  constexpr size_t kLds = (size_t)kWaves * Ring::kWaveBytes;
  static_assert(kLds >= sizeof(MergeLds) && kLds <= 160 * 1024, "LDS ring budget");
  auto fn = gqa_mfma_kernel<KV, PAGED, NT, 4, true>;
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
  if (tw == 1) {
    hipLaunchKernelGGL((gqa_mfma_kernel<KV, PAGED, true, 1, false>), grid, block, 0, stream, a);
  } else if (tw == 2) {
    if (nchunks == 1)
      hipLaunchKernelGGL((gqa_mfma_kernel<KV, PAGED, true, 2, false>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((gqa_mfma_kernel<KV, PAGED, false, 2, false>), grid, block, 0, stream, a);
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
