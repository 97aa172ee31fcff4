// Split-KV partial attention for a GQA group of up to 16 query heads on MFMA:
// the kernel template, shared by the translation units that instantiate it
// (partial_gqa_mfma.hip: accumulators in VGPRs; partial_gqa_mfma_tokens.hip:
// the one-wave two-token instances, accumulators in AGPRs).
//
// With 16 query heads sharing one KV head, every cached K and V element feeds
// 16 multiply-adds, which is more arithmetic per HBM byte than the fp32 vector
// ALUs can sustain for fp8 or MXFP4 caches.  The 16 heads of the group are
// exactly the 16-wide dimension of the gfx950 matrix instructions, so both
// contractions run on them:
//
//   S^T[token, head] = K_tile[token, :] . Q[head, :]     (4 MFMAs / 16 tokens)
//   O^T[dv, head]   += V_tile^T[dv, token] . P^T[token, head] (32 tokens, 8
//                                                        column blocks)
//
// Logits.  The cache's K elements are decoded to bf16 in registers (exact for
// every format: bf16, E4M3, and E2M1 times its E8M0 block scale) and multiply
// the bf16 query on v_mfma_f32_16x16x32_bf16, whose products are exact and
// whose accumulation is fp32-accurate.  (The block-scaled f8f6f4 instruction
// could take the fp8 / fp4 bytes as they are, but it sums its 128 products
// with an error of about 2^-13 of the largest one, which large logits turn
// into visible log-sum-exp errors.)  An fp8 slab's scale is folded into the
// log2 multiplier of the logits; the query carries its sign.
//
// Weights.  P = exp2(logit - running max) in fp32; the running sum of these
// fp32 weights gives the log-sum-exp.  The PV product takes P
//  * for fp8 and MXFP4 caches as fp16 (truncated, offset by 2^7 so that
//    weights down to 2^-31 of the largest are kept), against V decoded to
//    fp16 (exact for E4M3, and for E2M1 whenever the tile's block exponents
//    lie in [114, 140]; a tile outside that range takes the bf16 pair below),
//    one v_mfma_f32_16x16x32_f16 per block, and the output is normalized by
//    the sum of the same fp16 weights (one more MFMA against a ones operand),
//    so it is an exact convex combination of the cached values whose weights
//    are within 2^-10 (relative) of the softmax's;
//  * for bf16 caches as a bf16 pair hi + lo (two MFMAs), ~16 significant bits,
//    normalized by the fp32 sum.
//
// Work split: one workgroup of 4 waves per (shard j, request b, KV head,
// chunk of query tokens: one token for a single-token decode, two or four for
// a multi-token turn); wave w takes the shard's 32-token tiles w, w+4, w+8, ...
// and, for one token, keeps the loads of its next one (bf16) or three (fp8,
// MXFP4: smaller tiles) tiles in flight while computing the current one (fp8
// at one wave per SIMD, MXFP4 at two).  With enough shard units the one-wave
// split (SOLO below) replaces the four-wave one.  Several tokens share every
// loaded tile (see TW below).
// Lane (r, g) = (lane % 16, lane / 16):
//  * K: lane (r, g) loads token r of each 16-token half-tile, bytes
//    [64i + 16g, 64i + 16g + 16) of the row for each 16-byte load i, so each
//    load instruction reads 64 contiguous bytes of 16 rows.  MFMA chunk c of
//    the logits contracts the 8 dims Layout::chunk_d(c, g) of this lane's
//    bytes (and the query supplies the same dims).
//  * V: lane (r, g) loads columns [8r, 8r + 8) of the 8 tokens
//    {4g..4g+3, 16+4g..16+4g+3}, one full row per 16 lanes per instruction, and
//    regroups them with byte permutes into per-column token octets.
//  * The S^T output of the MFMA gives lane (n, g) head n at tokens
//    {4g+i, 16+4g+i}: exactly the P^T operand of the PV MFMA, so softmax state
//    (running max, partial sum) is per lane and needs no transposes; the O^T
//    accumulator of lane (n, g) is head n, dv in [32g, 32g + 32).
// The running max is only moved when a tile's max exceeds it by more than 2^8
// (in the exp2 domain); the stale max is exact algebra and keeps P <= 2^8
// (fp16 weights, offset by 2^7: <= 2^15).
// At the end the four waves' (max, sums, acc) states are merged through LDS
// and the normalized partial o and its natural-log lse are written.
#pragma once

#include <type_traits>

#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kD = 128;        // head width (Dqk = Dv)
constexpr int kTile = 32;      // tokens per wave iteration
constexpr float kLazyMax = 8.0f;
// fp16 weights are 2^kPOffset times exp2(logit - running max): at most 2^15
// (below fp16's largest, 65504) and no smaller than 2^7 for the largest
// weight, so fp16's smallest subnormal, 2^-24, is 2^-31 of it.
constexpr float kPOffset = 7.0f;
// MXFP4 V block exponents whose E2M1 values (0.5 .. 6 times 2^(E-127)) are
// normal fp16 numbers: E in [kVE16Lo, kVE16Lo + kVE16Span].
constexpr uint32_t kVE16Lo = 114;
constexpr uint32_t kVE16Span = 26;

__device__ __forceinline__ u32x4_t u4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4_t v = {a, b, c, d};
  return v;
}
__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8_t, u4(a, b, c, d));
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

// chunk_d(c, g): first of the 8 consecutive dims that lane group g supplies
// to MFMA chunk c of the logits (the dims its K loads hold, in order).
// bf16: 64 B of K per lane per half-tile (4 loads: dims 32i + 8g .. +7 of
// load i), 16 B of V per token.
// Occupancy of the one-token instances: kWavesPerEu, the waves per SIMD the
// registers are sized for; kLdsReserve, dynamic LDS reserved per workgroup
// (0: none; above half the CU's LDS it keeps one workgroup, i.e. one wave,
// per SIMD); kSoloWaves, the wave count from which one-wave shard groups
// replace the four-wave split (0: never); kSoloTokenUnits, the same for two
// to four query tokens, one wave per (shard, two-token chunk) (measured: from
// 1024 units on for fp8; for MXFP4, whose decode and matrix work per byte is
// twice fp8's, only from 8192 units on); kStash, the finished shard
// partials a one-wave group keeps in LDS before writing them out (each batch
// of stores a wave issues costs it about as long as its writes take to drain,
// tens of microseconds under a full read stream, because later loads are
// counted behind the stores).  Measured: the fp8 pass streams
// best at one wave per SIMD (two waves per SIMD do not share the issue
// fairly: one of them runs far ahead and the other finishes alone), the
// MXFP4 pass, with twice the arithmetic per byte, at two.
template <>
struct Layout<kBF16> {
  static constexpr int kWavesPerEu = 1;
  static constexpr int kLdsReserve = 0;
  static constexpr int kSoloWaves = 0;
  static constexpr int kSoloTokenUnits = 0;
  static constexpr int kStash = 1;
  static constexpr int kRing = 2;       // tiles held in registers (current + prefetched)
  static constexpr int kKLoads = 4;     // 16-byte K loads per lane per half-tile
  static constexpr int kVBytes = 16;    // V bytes per lane per token
  static constexpr int kRowBytes = 256;
  __device__ static constexpr int chunk_d(int c, int g) { return 32 * c + 8 * g; }
};
// fp8: lane (r, g) holds dims 16g .. 16g+15 and 64+16g .. 64+16g+15.
template <>
struct Layout<kFP8> {
  static constexpr int kWavesPerEu = 1;
  static constexpr int kLdsReserve = 96 * 1024;
  static constexpr int kSoloWaves = 1024;
  static constexpr int kSoloTokenUnits = 1024;
  static constexpr int kStash = 4;
  static constexpr int kRing = 4;
  static constexpr int kKLoads = 2;
  static constexpr int kVBytes = 8;
  static constexpr int kRowBytes = 128;
  __device__ static constexpr int chunk_d(int c, int g) { return 64 * (c >> 1) + 16 * g + 8 * (c & 1); }
};
// MXFP4: lane (r, g) holds dims 32g .. 32g+31 (one E8M0 block).
template <>
struct Layout<kMXFP4> {
  static constexpr int kWavesPerEu = 2;
  static constexpr int kLdsReserve = 0;
  static constexpr int kSoloWaves = 2048;
  static constexpr int kSoloTokenUnits = 8192;
  static constexpr int kStash = 2;
  static constexpr int kRing = 4;
  static constexpr int kKLoads = 1;
  static constexpr int kVBytes = 4;
  static constexpr int kRowBytes = 64;
  __device__ static constexpr int chunk_d(int c, int g) { return 32 * g + 8 * c; }
};

// V of the fp8 and MXFP4 caches reaches the registers coalesced, 16 bytes
// per lane per load (a 16-row half-tile is one load per lane for MXFP4, two
// for fp8, where the PV operand layout would need four single-token loads of
// 4 or 8 bytes: the address unit's time goes by load instruction, not by
// byte), and is regrouped through a per-wave LDS patch when its tile is
// computed.  Row stride in the patch: 32 pad bytes (fp8) put the four token
// groups a read instruction gathers on disjoint banks; with 16 (MXFP4) the
// reads still meet bank conflicts on a few percent of the cycles, and a
// conflict-free placement measured the same time.
template <int KV>
struct VPatch {
  static constexpr int kRow = Layout<KV>::kRowBytes + (KV == kMXFP4 ? 16 : 32);
  static constexpr int kHalf = 16 * kRow;            // one half-tile
  static constexpr int kWaveBytes = 2 * kHalf;       // a tile
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
// per: units of one request (shard or shard-group positions times Hkv).
__device__ __forceinline__ int64_t longest_first_unit(int64_t p, const PartialArgs& a, int per) {
  if (a.B <= 1 || a.B > 64) return p;
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

// One stashed shard partial in LDS: 16 rows (heads) of kD floats, padded to
// kStashRow, then the 16 lse values.
constexpr int kStashRow = kD + 4;
constexpr int kStashFloats = 16 * kStashRow + 16;
template <int KV>
constexpr size_t stash_bytes() { return (size_t)kWaves * Layout<KV>::kStash * kStashFloats * sizeof(float); }

// LDS of the final merge of the four waves' states: accumulators, running
// maxima, fp32 weight sums (for the lse) and the sums the accumulators are
// normalized by (the fp16 weights' for fp8 / MXFP4 caches).
struct MergeLds {
  float o[kWaves][16][kD + 4];
  float m[kWaves][16];
  float l[kWaves][16];
  float ln[kWaves][16];
};

// K operand of logits chunk c of half-tile u, decoded to bf16: the 8 dims
// Layout::chunk_d(c, g) of token 16u + r16 (fp8: unscaled codes; MXFP4: times
// the block's E8M0 scale, E = 0 taken as 0 and E = 255 as +inf).
template <int KV>
__device__ __forceinline__ bf16x8_t k_operand(const Raw<KV>& rw, int u, int c) {
  if constexpr (KV == kBF16) {
    return as_bf16x8(rw.k[u][4 * c], rw.k[u][4 * c + 1], rw.k[u][4 * c + 2], rw.k[u][4 * c + 3]);
  } else if constexpr (KV == kFP8) {
    const uint32_t w0 = rw.k[u][2 * c], w1 = rw.k[u][2 * c + 1];
    return as_bf16x8(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true)));
  } else {
    const uint32_t w = rw.k[u][c];
    const float sc = e8m0_to_f32_fast(rw.ks[u]);
    return as_bf16x8(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2)),
                     __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3)));
  }
}

// Whether every V block exponent of an MXFP4 tile decodes to normal fp16
// values (wave-uniform).
__device__ __forceinline__ bool v_fits_f16(const Raw<kMXFP4>& rw) {
  const bool ok = (rw.vs[0] - kVE16Lo) <= kVE16Span && (rw.vs[1] - kVE16Lo) <= kVE16Span;
  return __all(ok);
}

// V^T operands of the 8 16-column blocks of the PV product, decoded to fp16
// (F16) or bf16: f(blk, op) is called for each block as soon as its operand
// (four dwords) is ready.  The operand of block blk holds the lane's column of
// that block for the 8 tokens {4g + i, 16 + 4g + i}, in the k order of the
// P^T operand.  fp16 needs fp8 (E4M3 codes are fp16 numbers) or an MXFP4 tile
// that v_fits_f16; a bf16 cache is bf16 only.
// MXFP4: lane L of the wave holds the V exponent of (token 16u + L / 4,
// column block L % 4) in rw.vs[u]; vs_lane is the byte address (for
// ds_bpermute) of the lane holding this lane's block (r / 4) of token 4g.
template <int KV, bool F16, class F>
__device__ __forceinline__ void for_v_operands(const Raw<KV>& rw, uint32_t vs_lane, F&& f) {
  static_assert(!(F16 && KV == kBF16), "bf16 cache: bf16 V");
  if constexpr (KV == kBF16) {
    // rw.v[e][q] = columns (8 r16 + 2q, 8 r16 + 2q + 1) of token e
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const int q = blk / 2;
      const uint32_t sel = (blk & 1) ? 0x07060302u : 0x05040100u;
      f(blk, u4(perm(rw.v[1][q], rw.v[0][q], sel), perm(rw.v[3][q], rw.v[2][q], sel),
                perm(rw.v[5][q], rw.v[4][q], sel), perm(rw.v[7][q], rw.v[6][q], sel)));
    }
  } else if constexpr (KV == kMXFP4) {
    // the block scale of each of the lane's 8 tokens: token 16 (e / 4) + 4g +
    // e % 4 sits 4 (e % 4) lanes past token 4g
    float vsc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      vsc[e] = e8m0_to_f32_fast(
          (uint32_t)__builtin_amdgcn_ds_bpermute((int)(vs_lane + 16 * (e % 4)), (int)rw.vs[e / 4]));
    // one column pair q (blocks 2q, 2q + 1) at a time: cv[e] = columns
    // (8 r16 + 2q, 8 r16 + 2q + 1) of token e
    auto pair = [&](auto q_tag) {
      constexpr int q = decltype(q_tag)::value;
      uint32_t cv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (F16)
          cv[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(rw.v[e][0], vsc[e], q));
        else
          cv[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(rw.v[e][0], vsc[e], q));
      }
      f(2 * q, u4(perm(cv[1], cv[0], 0x05040100u), perm(cv[3], cv[2], 0x05040100u),
                  perm(cv[5], cv[4], 0x05040100u), perm(cv[7], cv[6], 0x05040100u)));
      f(2 * q + 1, u4(perm(cv[1], cv[0], 0x07060302u), perm(cv[3], cv[2], 0x07060302u),
                      perm(cv[5], cv[4], 0x07060302u), perm(cv[7], cv[6], 0x07060302u)));
    };
    pair(std::integral_constant<int, 0>{});
    pair(std::integral_constant<int, 1>{});
    pair(std::integral_constant<int, 2>{});
    pair(std::integral_constant<int, 3>{});
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
          if constexpr (F16) {
            lo[rr] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x2, 1.0f, false));
            hi[rr] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x2, 1.0f, true));
          } else {
            lo[rr] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x2, 1.0f, false));
            hi[rr] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x2, 1.0f, true));
          }
        }
        f(4 * q + s2, u4(lo[0], lo[1], lo[2], lo[3]));
        f(4 * q + s2 + 1, u4(hi[0], hi[1], hi[2], hi[3]));
      }
    }
  }
}

// Weights of one token on one tile in the formats of the PV product.
struct Weights {
  u32x4_t h;    // fp16 weights (F16 path) or the bf16 upper halves (pair path)
  u32x4_t lo;   // pair path: the bf16 remainders
};

// One 16-column block of O^T += V^T P^T (or, against ones_operand, the sum of
// the weights): fp16 weights (F16) or the bf16 pair.
template <bool F16>
__device__ __forceinline__ f32x4_t pv_mfma(const u32x4_t& v, const Weights& w, f32x4_t acc) {
  if constexpr (F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, v), __builtin_bit_cast(f16x8_t, w.h),
                                                  acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, v), __builtin_bit_cast(bf16x8_t, w.h),
                                                  acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, v),
                                                   __builtin_bit_cast(bf16x8_t, w.lo), acc, 0, 0, 0);
  }
}
// The ones operand of the weight-sum product (fp16 or bf16 1.0 in every element).
template <bool F16>
__device__ __forceinline__ u32x4_t ones_operand() {
  const uint32_t one = F16 ? 0x3C003C00u : 0x3F803F80u;
  return u4(one, one, one, one);
}

// PAGED: rows are found through the block table (paged cache layout).
// NT: cache loads carry the non-temporal hint: every cache byte is read once
// when one token chunk covers all query tokens.  With several chunks each
// chunk reads the shard's rows, the loads are plain, and the later chunks of
// a shard find them in the caches.
// TW: query tokens per workgroup.  Each wave loads a tile (and decodes its K
// and V) once and runs the logits, softmax and PV product of each of the TW
// tokens on it; every token keeps its own Q operands, softmax state and
// accumulators.
// LDSRING: the tiles ahead wait in an LDS ring filled by direct-to-LDS loads
// (Ring, bf16 cache) instead of in registers, which leaves the registers to the
// tokens and keeps several tiles in flight at one wave per SIMD.
// SOLO: each wave takes a whole unit and chunk (wave 4 blockIdx + wave: unit
// w / nchunks, a group of solo_shards consecutive shards, and chunk
// w % nchunks of TW query tokens) and streams its tiles in order, then writes
// the partials: no barrier.  One token: the partials of a group wait in LDS
// slots and go out together at the end; TW tokens: one shard per wave,
// written from registers at the end.  Used when
// there are enough units to keep every SIMD streaming, where the four-wave
// merge and the per-workgroup set-up of the default split cost more than
// they save.
template <int KV, bool PAGED, bool NT, int TW, bool LDSRING, bool SOLO>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(TW == 1 ? Layout<KV>::kWavesPerEu : 1)))
void gqa_mfma_kernel(PartialArgs a) {
  using Lay = Layout<KV>;
  constexpr int64_t ROW = Lay::kRowBytes;
  constexpr int kRing = TW > 1 ? 2 : Lay::kRing;
  // fp16 weights against fp16 V (fp8, MXFP4), normalized by their own sum
  constexpr bool F16PV = KV != kBF16;
  constexpr int NACC = F16PV ? 9 : 8;      // PV accumulators (+ the weight sum)
  constexpr float POFF = F16PV ? kPOffset : 0.0f;

  static_assert(!SOLO || !LDSRING, "one-wave units: register ring");
  // tile i of a wave's sequence is tile first + i * kStride of its shard
  constexpr int kStride = SOLO ? 1 : kWaves;
  MergeLds* mrg = nullptr;
  uint32_t ring_lds = 0;   // LDSRING: LDS address of this wave's slots
  if constexpr (LDSRING) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
    mrg = reinterpret_cast<MergeLds*>(dyn_lds);   // reused once the ring is drained
    ring_lds = (uint32_t)(uintptr_t)(lds_u8*)dyn_lds +
               (uint32_t)(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * Ring::kWaveBytes);
  } else if constexpr (!SOLO) {
    __shared__ MergeLds st;
    mrg = &st;
  }
  // fp8 / MXFP4, one token, register ring: V loaded coalesced, regrouped
  // through this wave's LDS patch (VPatch).  (The two-token instances, whose
  // longer tile computation covers the loads, measured slower with it.)
  constexpr bool VT = KV != kBF16 && !LDSRING && TW == 1;
  uint32_t vt_lds = 0;
  if constexpr (VT) {
    __shared__ __attribute__((aligned(16))) uint8_t vt_st[kWaves * VPatch<KV>::kWaveBytes];
    vt_lds = (uint32_t)(uintptr_t)(lds_u8*)vt_st +
             (uint32_t)(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * VPatch<KV>::kWaveBytes);
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
  // SOLO: a unit is a group of solo_shards consecutive shards of one (request,
  // KV head); njp groups per (request, KV head)
  const int njp = SOLO ? (a.kvp + a.solo_shards - 1) / a.solo_shards : a.kvp;
  if constexpr (SOLO) {
    // the chunks of a unit are consecutive waves of one workgroup, so the
    // later ones find the unit's rows in the caches
    const int64_t w = (int64_t)blockIdx.x * kWaves + wave;
    unit = w / nchunks;
    chunk = (int)(w - unit * nchunks);
    if (unit >= (int64_t)njp * a.B * a.Hkv) return;   // the whole wave: no barrier follows
  } else {
    if (!unit_token(blockIdx.x, (int64_t)a.kvp * a.B * a.Hkv, nchunks, &unit, &chunk)) return;
  }
  unit = longest_first_unit(unit, a, njp * a.Hkv);
  const int first = SOLO ? 0 : wave;                // first tile of this wave
  const int kvh = (int)(unit % a.Hkv);
  const int b = (int)(unit / a.Hkv % a.B);
  // shard (SOLO: first shard of the group)
  const int j = (int)(unit / ((int64_t)a.Hkv * a.B)) * (SOLO ? a.solo_shards : 1);
  const int qt0 = chunk * TW;                       // first query token of the chunk
  const int nq = a.T - qt0 < TW ? a.T - qt0 : TW;   // tokens of the chunk that exist

  // The rows the shard holds are [s0, s1); token i of the chunk sees rows
  // [s0, s1t[i]) (its causal cut).  Later tokens see more, so the last one
  // bounds the rows read; tokens past the end of T see none.
  const int64_t L = a.seq_lens[b];
  const ShardSpan span = shard_span(a.layout, L, a.T, qt0 + nq - 1, a.S_max, a.kvp, a.B, a.Hkv, j, b, kvh);
  // the token rows streamed: [s0, s1) (SOLO: reset for each run of shards)
  int64_t s0 = span.s0, s1 = span.s1;
  int64_t s1t[TW];
#pragma unroll
  for (int i = 0; i < TW; ++i)
    s1t[i] = i >= nq ? s0 : (i == nq - 1 ? s1 : shard_span(a.layout, L, a.T, qt0 + i, a.S_max, a.kvp, a.B, a.Hkv,
                                                            j, b, kvh).s1);
  int64_t slab = span.slab;                        // cache block of this shard
  const int64_t bh = (int64_t)b * a.Hkv + kvh;     // fp8 scales are per (request, KV head)

  // The cache arrays are viewed as rows of ROW bytes (scales: kD/32 bytes).
  // Contiguous and sharded layouts: token t of this shard is row
  // slab * S_max + t, so pointers start at the slab; paged: rows come from
  // the block table (phys_row) and pointers start at the pool.
  const uint8_t* kdata = nullptr;
  const uint8_t* vdata = nullptr;
  const uint8_t* ksdata = nullptr;
  const uint8_t* vsdata = nullptr;
  auto set_slab = [&](int64_t sl) {
    slab = sl;
    const int64_t row0 = PAGED ? 0 : sl * a.S_max;
    kdata = static_cast<const uint8_t*>(a.k) + row0 * ROW;
    vdata = static_cast<const uint8_t*>(a.v) + row0 * ROW;
    if constexpr (KV == kMXFP4) {
      ksdata = static_cast<const uint8_t*>(a.k_scale) + row0 * (kD / 32);
      vsdata = static_cast<const uint8_t*>(a.v_scale) + row0 * (kD / 32);
    }
  };
  set_slab(span.slab);
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
  // raw logit -> log2 domain.  A negative fp8 K scale flips the sign of
  // every logit of the slab: the query operands carry that sign, so the raw
  // products already are the signed logits and c2 stays >= 0.
  const float c2 = a.scale_log2 * fabsf(kscale);
  const uint32_t qsign = kscale < 0.0f ? 0x80008000u : 0u;

  // Q^T operands of each token of the chunk (a token past the end of T loads
  // the last one's): lane (n, g) holds head n, the 8 dims chunk_d(c, g).  A
  // group of G < 16 heads fills the first G of the 16 MFMA columns; the other
  // columns get zero queries and their outputs are never written.
  const int G = a.Hq / a.Hkv;
  const bool head_ok = r16 < G;
  bf16x8_t qop[TW][4];
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    const int qt = qt0 + (i < nq ? i : nq - 1);
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + (((int64_t)b * a.T + qt) * a.Hq + kvh * G + (head_ok ? r16 : 0)) * kD;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 v = *reinterpret_cast<const uint4*>(qrow + Lay::chunk_d(c, g));
      if (!head_ok) v = make_uint4(0u, 0u, 0u, 0u);
      qop[i][c] = as_bf16x8(v.x ^ qsign, v.y ^ qsign, v.z ^ qsign, v.w ^ qsign);
    }
  }

  f32x4_t acc[TW][NACC];
  float m2[TW];    // running max of this lane's head (log2 domain)
  float lsum[TW];  // partial sum of the fp32 weights over this lane's tokens
#pragma unroll
  for (int i = 0; i < TW; ++i) {
#pragma unroll
    for (int k = 0; k < NACC; ++k) acc[i][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m2[i] = -INFINITY;
    lsum[i] = 0.0f;
  }

  int64_t last = s1 - 1;
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
        if constexpr (VT) {
          // coalesced: byte 16 lane (+ 1024) of the half-tile, i.e. row
          // 16 lane / ROW, regrouped by v_regroup when the tile is computed
          const u32x4_t v0 = buf_load16<NT>(rv, (uint32_t)(16 * lane));
          if constexpr (Lay::kVBytes == 4) {
#pragma unroll
            for (int w = 0; w < 4; ++w) rw.v[4 * u + w][0] = v0[w];
          } else {
            const u32x4_t v1 = buf_load16<NT>(rv, (uint32_t)(16 * lane + 1024));
            rw.v[4 * u][0] = v0[0];
            rw.v[4 * u][1] = v0[1];
            rw.v[4 * u + 1][0] = v0[2];
            rw.v[4 * u + 1][1] = v0[3];
            rw.v[4 * u + 2][0] = v1[0];
            rw.v[4 * u + 2][1] = v1[1];
            rw.v[4 * u + 3][0] = v1[2];
            rw.v[4 * u + 3][1] = v1[3];
          }
        } else
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
  // kop holds the decoded K operands (TW > 1: decoded once for all tokens);
  // for one token each operand is decoded next to its MFMA.
  auto logits = [&](const Raw<KV>& rw, const bf16x8_t (&kop)[2][4], int i, float (&x)[8]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if constexpr (TW == 1)
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand<KV>(rw, u, c), qop[i][c], s, 0, 0, 0);
        else
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[u][c], qop[i][c], s, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * u + e] = s[e];
    }
  };
  // Max of the lane's 8 logits of its head, in the log2 domain.  Whether the
  // running max must move is decided on these lane maxima (any lane over its
  // head's max + 2^kLazyMax); only then is the head's tile max reduced over
  // its 4 lane groups, so all 4 keep the same running max.  (A lane whose
  // logits are all masked gives NaN when c2 = 0: no lane is over the max
  // then, and the reductions skip NaN.)
  auto lane_max2 = [&](const float (&x)[8]) {
    float tmax = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, x[e]);
    return tmax * c2;
  };
  // Move the running max to mn, rescaling the state.
  auto rescale = [&](float& m, float& l, f32x4_t (&o)[NACC], float mn) {
    const float al = fast_exp2(m - mn);
    l *= al;
#pragma unroll
    for (int i = 0; i < NACC; ++i) o[i] *= al;
    m = mn;
  };
  // Softmax weights P = 2^(x c2 - m + POFF) (0 for masked logits), added to
  // the fp32 running sum and packed for the PV product: F16, as fp16
  // (truncated); otherwise (bf16 caches, MXFP4 tiles outside the fp16 range)
  // as the bf16 pair: hi keeps the upper 16 bits of each fp32 weight (exact),
  // lo the remainder rounded to bf16, so hi + lo carries ~16 significant bits.
  auto weights = [&](const float (&x)[8], float m, float& l, Weights& w, auto f16_tag, auto mask_tag) {
    constexpr bool F16 = decltype(f16_tag)::value;
    constexpr bool MASK = decltype(mask_tag)::value;
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = fast_exp2(fmaf(x[e], c2, POFF - m));
      if constexpr (MASK) p[e] = (x[e] == -INFINITY) ? 0.0f : p[e];
      l += p[e];
    }
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      if constexpr (F16) {
        ph[rr] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(p[2 * rr], p[2 * rr + 1]));
      } else {
        const uint32_t b0 = __float_as_uint(p[2 * rr]), b1 = __float_as_uint(p[2 * rr + 1]);
        ph[rr] = perm(b1, b0, 0x07060302u);
        pl[rr] = pack_bf16(p[2 * rr] - __uint_as_float(b0 & 0xFFFF0000u),
                           p[2 * rr + 1] - __uint_as_float(b1 & 0xFFFF0000u));
      }
    }
    w.h = u4(ph[0], ph[1], ph[2], ph[3]);
    if constexpr (!F16) w.lo = u4(pl[0], pl[1], pl[2], pl[3]);
  };
  // Whether this tile's PV product runs on fp16 (wave-uniform).
  auto tile_f16 = [&](const Raw<KV>& rw) -> bool {
    if constexpr (KV == kFP8) return true;
    else if constexpr (KV == kMXFP4) return v_fits_f16(rw);
    else return false;
  };

  // Every token of the chunk on one tile, phase by phase: the K operands
  // (decoded once for all tokens when TW > 1) for the logits of all tokens,
  // one rescale check, the weights of all, then V decoded block by block
  // straight into every token's PV product (and the weight sums).  The
  // tokens' independent MFMA chains interleave, and neither all K nor all V
  // operands are held at once.  MASK: token i sees the tile's rows below
  // nv[i] only (none when nv[i] <= 0).
  auto tokens_tile = [&](const Raw<KV>& rw, const int (&nv)[TW], auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    float x[TW][8];
    {
      bf16x8_t kop[2][4];
      if constexpr (TW > 1) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int c = 0; c < 4; ++c) kop[u][c] = k_operand<KV>(rw, u, c);
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
    if constexpr (F16PV) {
      if (tile_f16(rw)) {
        Weights wf[TW];
#pragma unroll
        for (int i = 0; i < TW; ++i) weights(x[i], m2[i], lsum[i], wf[i], std::true_type{}, mask_tag);
        for_v_operands<KV, true>(rw, vs_lane, [&](int blk, const u32x4_t& v) {
#pragma unroll
          for (int i = 0; i < TW; ++i) acc[i][blk] = pv_mfma<true>(v, wf[i], acc[i][blk]);
        });
#pragma unroll
        for (int i = 0; i < TW; ++i) acc[i][8] = pv_mfma<true>(ones_operand<true>(), wf[i], acc[i][8]);
        return;
      }
    }
    // bf16 V against the bf16 pair
    Weights wb[TW];
#pragma unroll
    for (int i = 0; i < TW; ++i) weights(x[i], m2[i], lsum[i], wb[i], std::false_type{}, mask_tag);
    for_v_operands<KV, false>(rw, vs_lane, [&](int blk, const u32x4_t& v) {
#pragma unroll
      for (int i = 0; i < TW; ++i) acc[i][blk] = pv_mfma<false>(v, wb[i], acc[i][blk]);
    });
    if constexpr (F16PV) {
#pragma unroll
      for (int i = 0; i < TW; ++i) acc[i][8] = pv_mfma<false>(ones_operand<false>(), wb[i], acc[i][8]);
    }
  };

  // MASK: the tile runs past the shard end, or past a token's cut: rows at or
  // past a token's cut get weight 0.
  using Masked = std::true_type;      // compute: rows past a token's cut get weight 0
  using Unmasked = std::false_type;
  using FullTile = std::true_type;    // load: every row of the tile inside the shard
  using PartTile = std::false_type;
  using Clamped = std::true_type;     // issue: rows clamped to the shard, lane by lane
  using Unclamped = std::false_type;
  // The V registers of a full tile (loaded coalesced) through the wave's LDS
  // patch into the PV operand layout: rw.v[e] = columns kVBytes r16 .. of
  // token 16 (e / 4) + 4g + e % 4, as the partial-tile loads give them.
  // Wave-local: the wave's LDS operations run in order, no barrier.
  auto v_regroup = [&](const Raw<KV>& rw) {
    using P = VPatch<KV>;
    Raw<KV> rt = rw;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // lane's 16 bytes at row 16 lane / ROW, byte 16 lane % ROW (+ 8 rows)
      const uint32_t wr = vt_lds + (uint32_t)(u * P::kHalf + (16 * lane / ROW) * P::kRow + (16 * lane) % ROW);
      if constexpr (Lay::kVBytes == 4) {
        *(lds_u32x4*)(uintptr_t)wr = u4(rw.v[4 * u][0], rw.v[4 * u + 1][0], rw.v[4 * u + 2][0], rw.v[4 * u + 3][0]);
      } else {
        *(lds_u32x4*)(uintptr_t)wr = u4(rw.v[4 * u][0], rw.v[4 * u][1], rw.v[4 * u + 1][0], rw.v[4 * u + 1][1]);
        *(lds_u32x4*)(uintptr_t)(wr + 8 * P::kRow) =
            u4(rw.v[4 * u + 2][0], rw.v[4 * u + 2][1], rw.v[4 * u + 3][0], rw.v[4 * u + 3][1]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t rd = vt_lds + (uint32_t)((e / 4) * P::kHalf + (4 * g + e % 4) * P::kRow + Lay::kVBytes * r16);
      if constexpr (Lay::kVBytes == 4) {
        rt.v[e][0] = *(const lds_u32*)(uintptr_t)rd;
      } else {
        const u32x2_t v = *(const lds_u32x2*)(uintptr_t)rd;
        rt.v[e][0] = v[0];
        rt.v[e][1] = v[1];
      }
    }
    return rt;
  };
  auto compute = [&](const Raw<KV>& rw_in, int tile, auto mask_tag) {
    // full tiles (Unmasked) of fp8 / MXFP4 come coalesced (VT: one token)
    const Raw<KV> rw = [&] {
      if constexpr (VT && !decltype(mask_tag)::value) return v_regroup(rw_in);
      else return rw_in;
    }();
    const int64_t base = s0 + (int64_t)tile * kTile;
    int nv[TW];
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      const int64_t n = s1t[i] - base;         // wave-uniform
      nv[i] = n < 0 ? 0 : (n > kTile ? kTile : (int)n);
    }
    if constexpr (TW == 1 && decltype(mask_tag)::value) {
      tokens_tile(rw, nv, Masked{});
    } else if constexpr (TW == 1) {
      tokens_tile(rw, nv, Unmasked{});
    } else {
      if (nv[0] == kTile)                        // every token sees the whole tile
        tokens_tile(rw, nv, Unmasked{});
      else
        tokens_tile(rw, nv, Masked{});
    }
  };

  int nfull = (int)((s1 - s0) / kTile);
  int ntiles = (int)((s1 - s0 + kTile - 1) / kTile);
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
    // Stream over this wave's full tiles of [s0, s1) with kRing register
    // buffers: the loads of the next kRing-1 tiles are in flight while a tile
    // is computed.  (With several query tokens a tile takes several times
    // longer to compute, so one tile ahead is enough and leaves the registers
    // to the tokens.)  The next loads are always issued (clamped to the last
    // full tile) so the waits stay static.  A partial last tile is handled
    // once, after the ring.  on_tile(tile) runs before each tile's compute.
    auto stream_tiles = [&](auto&& on_tile) {
      if (nfull > 0) {
        auto clampt = [&](int t) { return t < nfull - 1 ? t : nfull - 1; };
        int tile = first;
        // rb[k] holds tile first + (n kRing + k) kStride; the loop body is
        // unrolled kRing times so that every buffer index is a constant
        Raw<KV> rb[kRing];
#pragma unroll
        for (int k = 0; k < kRing - 1; ++k) load(rb[k], clampt(tile + k * kStride), FullTile{});
        bool more = tile < nfull;
        while (more) {
#pragma unroll
          for (int k = 0; k < kRing; ++k) {
            if (more) {
              load(rb[(k + kRing - 1) % kRing], clampt(tile + (kRing - 1) * kStride), FullTile{});
              on_tile(tile);
              compute(rb[k], tile, Unmasked{});
              tile += kStride;
              more = tile < nfull;
            }
          }
        }
      }
      if (nfull < ntiles && (SOLO || nfull % kWaves == wave)) {
        Raw<KV> rt;
        load(rt, nfull, PartTile{});
        on_tile(nfull);
        compute(rt, nfull, Masked{});
      }
    };
    if constexpr (!SOLO) {
      stream_tiles([](int) {});
    } else if constexpr (TW > 1) {
      // ---- one wave, one shard, all query tokens: write each token's
      // partial from the registers (layout as in finalize below)
      stream_tiles([](int) {});
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        if (i >= nq) break;
        const float lw = rows4_sum(lsum[i]);
        const bool empty = m2[i] == -INFINITY;
        const float ln = F16PV ? acc[i][NACC - 1][0] : lw;
        const float inv = empty ? 0.0f : vscale / ln;
        if (head_ok) {
          const int64_t orow = (((int64_t)j * a.B + b) * a.T + qt0 + i) * a.Hq + kvh * G + r16;
          float4* dst = reinterpret_cast<float4*>(a.o_part + orow * kD + 32 * g);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int e = k / 2, b0 = 4 * (k % 2);
            dst[k] = make_float4(acc[i][b0][e] * inv, acc[i][b0 + 1][e] * inv, acc[i][b0 + 2][e] * inv,
                                 acc[i][b0 + 3][e] * inv);
          }
          if (g == 0) a.lse_part[orow] = empty ? -INFINITY : (m2[i] - POFF + fast_log2(lw)) * kLn2;
        }
      }
      return;
    } else {
      // ---- one wave per group of shards j .. j1 - 1.  finalize(js) writes
      // shard js's partial from this wave's state and resets the state.  Lane
      // (n, g) holds head n, dv = 32g + 8e + blk in acc[0][blk][e], so float4
      // k of its 32 columns is acc[0][4 (k % 2) + i][k / 2], i < 4.
      // Finished partials wait in this wave's kStash LDS slots and go out in
      // one batch of stores at the end (a group has at most kStash shards).
      extern __shared__ __attribute__((aligned(16))) float stash_lds[];
      constexpr int kSlots = Layout<KV>::kStash;
      float* const my_stash = stash_lds + wave * kSlots * kStashFloats;
      int nstash = 0;
      uint64_t stash_js = 0;   // shard of slot s in bits [16s, 16s + 16)
      auto flush = [&]() {
        for (int sl = 0; sl < nstash; ++sl) {
          const int js = (int)((stash_js >> (16 * sl)) & 0xFFFFu);
          const float* src = my_stash + sl * kStashFloats;
          if (!head_ok) continue;
          const int64_t orow = (((int64_t)js * a.B + b) * a.T + qt0) * a.Hq + kvh * G + r16;
          float4* dst = reinterpret_cast<float4*>(a.o_part + orow * kD + 32 * g);
#pragma unroll
          for (int k = 0; k < 8; ++k) dst[k] = *reinterpret_cast<const float4*>(src + r16 * kStashRow + 32 * g + 4 * k);
          if (g == 0) a.lse_part[orow] = src[16 * kStashRow + r16];
        }
        nstash = 0;
        stash_js = 0;
      };
      // finalize(js): shard js's partial from this wave's state into the next
      // stash slot, and the state reset.  Lane (n, g) holds head n,
      // dv = 32g + 8e + blk in acc[0][blk][e], so float4 k of its 32 columns is
      // acc[0][4 (k % 2) + i][k / 2], i < 4.
      auto finalize = [&](int js) {
        const float lw = rows4_sum(lsum[0]);
        const bool empty = m2[0] == -INFINITY;
        const float ln = F16PV ? acc[0][NACC - 1][0] : lw;
        const float inv = empty ? 0.0f : vscale / ln;
        float* slot = my_stash + nstash * kStashFloats;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int e = k / 2, b0 = 4 * (k % 2);
          *reinterpret_cast<float4*>(slot + r16 * kStashRow + 32 * g + 4 * k) =
              make_float4(acc[0][b0][e] * inv, acc[0][b0 + 1][e] * inv, acc[0][b0 + 2][e] * inv,
                          acc[0][b0 + 3][e] * inv);
        }
        if (g == 0) slot[16 * kStashRow + r16] = empty ? -INFINITY : (m2[0] - POFF + fast_log2(lw)) * kLn2;
        stash_js |= (uint64_t)js << (16 * nstash);
        ++nstash;   // at most solo_shards <= kSlots finalizations per wave
#pragma unroll
        for (int k = 0; k < NACC; ++k) acc[0][k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m2[0] = -INFINITY;
        lsum[0] = 0.0f;
      };
      auto span_of = [&](int js) { return shard_span(a.layout, L, 1, 0, a.S_max, a.kvp, a.B, a.Hkv, js, b, kvh); };
      const int j1 = j + a.solo_shards < a.kvp ? j + a.solo_shards : a.kvp;
      // Consecutive shards of a contiguous or paged cache are one run of token
      // positions, streamed without a break when every shard boundary is a
      // tile boundary (shard length a multiple of the tile); otherwise, and
      // for sharded layouts (one slab per shard), shard by shard.
      bool one_run = a.layout == kContiguous || a.layout == kPaged;
      if (one_run) {
        const int64_t Lc = L < 0 ? 0 : (L > a.S_max ? a.S_max : L);
        const int64_t per = (Lc + a.kvp - 1) / a.kvp;
        one_run = ((per + 15) / 16 * 16) % kTile == 0;
      }
      for (int jj = j; jj < j1;) {
        const int je = one_run ? j1 : jj + 1;
        const ShardSpan sa = span_of(jj);
        s0 = sa.s0;
        s1 = je == jj + 1 ? sa.s1 : span_of(je - 1).s1;
        s1t[0] = s1;
        last = s1 - 1;
        nfull = (int)((s1 - s0) / kTile);
        ntiles = (int)((s1 - s0 + kTile - 1) / kTile);
        set_slab(sa.slab);
        int jcur = jj;
        int64_t bound = sa.s1;   // end of shard jcur
        stream_tiles([&](int tile) {
          const int64_t base = s0 + (int64_t)tile * kTile;
          while (base >= bound) {   // the tile starts a later shard
            finalize(jcur);
            ++jcur;
            bound = span_of(jcur).s1;
          }
        });
        for (; jcur < je; ++jcur) finalize(jcur);
        jj = je;
      }
      flush();
      return;
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
      // F16PV: the sum of the fp16 weights, the same in every element of the
      // weight-sum accumulator of head r16
      mrg->ln[wave][r16] = F16PV ? acc[i][NACC - 1][0] : lw;
    }
    __syncthreads();
    const int64_t orow0 = (((int64_t)j * a.B + b) * a.T + qt0 + i) * a.Hq + kvh * G;   // o_part / lse_part row
    const int tid = threadIdx.x;
    for (int idx = tid; idx < G * kD; idx += kThreads) {
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
          lt += mrg->ln[w][n] * f;
          ot += mrg->o[w][n][d] * f;
        }
        o = ot / lt * vscale;
      }
      a.o_part[(orow0 + n) * kD + d] = o;
    }
    if (tid < G) {
      float M = mrg->m[0][tid];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mrg->m[w][tid]);
      float lse = -INFINITY;
      if (M != -INFINITY) {
        float lt = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) lt += mrg->l[w][tid] * rescale_weight(mrg->m[w][tid], M);
        lse = (M - POFF + fast_log2(lt)) * kLn2;
      }
      a.lse_part[orow0 + tid] = lse;
    }
  }
}

}  // namespace
}  // namespace kvd
