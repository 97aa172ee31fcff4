// Device-side helpers shared by the libkvd kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvd {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum KvFormat : int { kF32 = 0, kBF16 = 1, kFP8 = 2, kMXFP4 = 3 };

// Bytes of one cached element (MXFP4 counts half a byte: use row bytes).
template <int KV>
struct KvTraits;
template <>
struct KvTraits<kF32> { static constexpr int kBitsPerElem = 32; };
template <>
struct KvTraits<kBF16> { static constexpr int kBitsPerElem = 16; };
template <>
struct KvTraits<kFP8> { static constexpr int kBitsPerElem = 8; };
template <>
struct KvTraits<kMXFP4> { static constexpr int kBitsPerElem = 4; };

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// E8M0 block exponent -> fp32 scale 2^(E-127).  E = 0 is the subnormal
// 2^-127 and E = 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  float s = __uint_as_float(e << 23);
  s = (e == 0u) ? __uint_as_float(0x00400000u) : s;
  s = (e == 255u) ? __uint_as_float(0x7FC00000u) : s;
  return s;
}

// E8M0 -> fp32 as a bare exponent shift, for the matrix-core kernels: exact
// for E in [1, 254]; E = 0 gives 0 instead of 2^-127 (every element of such a
// block is below 6 * 2^-127, under fp32's normal range) and E = 255 (NaN)
// gives +inf, so a NaN block scale yields non-finite results.
__device__ __forceinline__ float e8m0_to_f32_fast(uint32_t e) { return __uint_as_float(e << 23); }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) loads of cache bytes.  Every cached byte is read
// once per call, so the loads carry the non-temporal hint; on MI355X this is
// what lets a read stream approach HBM peak (regular loads plateau ~10%
// lower).  NT = false gives plain loads, for bytes that several workgroups
// read (the query tokens of a multi-token turn), which the caches should
// keep.  p must be aligned to the access size.
template <bool NT = true>
__device__ __forceinline__ u32x4_t stream_load16(const uint8_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  else return *reinterpret_cast<const u32x4_t*>(p);
}
template <bool NT = true>
__device__ __forceinline__ u32x2_t stream_load8(const uint8_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  else return *reinterpret_cast<const u32x2_t*>(p);
}
template <bool NT = true>
__device__ __forceinline__ uint32_t stream_load4(const uint8_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  else return *reinterpret_cast<const uint32_t*>(p);
}
template <bool NT = true>
__device__ __forceinline__ uint32_t stream_load1(const uint8_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// s_waitcnt immediate that waits until at most n vector memory operations
// remain in flight (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4 and
// lgkmcnt 11:8 left at their maxima).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// One direct-to-LDS 16-byte load per active lane: global address sbase + voff
// into LDS address M0 + 16 * lane, with the non-temporal hint when NT (bytes
// read once).  Inline asm, so the compiler does not take later LDS reads as
// aliasing it (it would wait for every load in flight, including the prefetch
// of the next tiles); the waits are explicit.  M0 belongs to the compiler, so
// it is saved and restored around the load.
template <bool NT>
__device__ __forceinline__ void lds_dma16(uint32_t m0, const uint8_t* sbase, uint32_t voff) {
  uint32_t m0_saved;
  if constexpr (NT) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(m0_saved)
        : "s"(m0), "v"(voff), "s"(sbase)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(m0_saved)
        : "s"(m0), "v"(voff), "s"(sbase)
        : "memory");
  }
}

// The same with a per-lane 64-bit global address (rows clamped lane by lane).
__device__ __forceinline__ void lds_dma16_at(uint32_t m0, const uint8_t* addr) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "s"(m0), "v"(addr)
      : "memory");
}

// Load N bytes (N in {4, 8, 16, 32, 64}) from a 4-byte-aligned (N >= 16:
// 16-byte aligned) global address into N/4 dwords, streaming.
template <int N>
__device__ __forceinline__ void load_dwords(const uint8_t* __restrict__ p, uint32_t* w) {
  static_assert(N % 4 == 0 && N >= 4, "whole dwords only");
  if constexpr (N >= 16) {
#pragma unroll
    for (int i = 0; i < N / 16; ++i) {
      const u32x4_t v = stream_load16(p + 16 * i);
      w[4 * i + 0] = v[0];
      w[4 * i + 1] = v[1];
      w[4 * i + 2] = v[2];
      w[4 * i + 3] = v[3];
    }
  } else if constexpr (N == 8) {
    const u32x2_t v = stream_load8(p);
    w[0] = v[0];
    w[1] = v[1];
  } else {
    w[0] = stream_load4(p);
  }
}

// Decode EPL consecutive elements held in dwords w (format KV) to fp32.
// fp8 scales are applied by the caller; the MXFP4 block scale is applied here.
template <int KV, int EPL>
__device__ __forceinline__ void decode_elems(const uint32_t* w, float mx_scale, float* out) {
  if constexpr (KV == kF32) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[e] = __uint_as_float(w[e]);
  } else if constexpr (KV == kBF16) {
#pragma unroll
    for (int i = 0; i < EPL / 2; ++i) {
      out[2 * i] = bf16_lo(w[i]);
      out[2 * i + 1] = bf16_hi(w[i]);
    }
  } else if constexpr (KV == kFP8) {
#pragma unroll
    for (int i = 0; i < EPL / 4; ++i) {
      auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
      auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
      out[4 * i + 0] = lo[0];
      out[4 * i + 1] = lo[1];
      out[4 * i + 2] = hi[0];
      out[4 * i + 3] = hi[1];
    }
  } else {
    static_assert(KV == kMXFP4, "format");
#pragma unroll
    for (int i = 0; i < EPL / 8; ++i) {
      auto b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], mx_scale, 0);
      auto b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], mx_scale, 1);
      auto b2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], mx_scale, 2);
      auto b3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], mx_scale, 3);
      out[8 * i + 0] = b0[0];
      out[8 * i + 1] = b0[1];
      out[8 * i + 2] = b1[0];
      out[8 * i + 3] = b1[1];
      out[8 * i + 4] = b2[0];
      out[8 * i + 5] = b2[1];
      out[8 * i + 6] = b3[0];
      out[8 * i + 7] = b3[1];
    }
  }
}

// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the result.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppRowHalfMirror>(v);
  v += dpp<kDppRowMirror>(v);
  return v;
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kDppQuadXor1>(v));
  v = fmaxf(v, dpp<kDppQuadXor2>(v));
  v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp<kDppRowMirror>(v));
  return v;
}

// Reductions over the four 16-lane rows (lanes l, l^16, l^32, l^48), on the
// gfx950 row-swap permutes: swapping a value with itself between row pairs
// leaves each lane holding one value of each pair in the two results, so
// op(first, second) is the pairwise reduction, identical in both rows.
__device__ __forceinline__ float rows4_max(float v) {
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
  auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(s[0]) + __uint_as_float(s[1]);
  auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Weight 2^(m - M) of a running state with max m inside a merged max M
// (zero when the state has seen no token, m = -inf).
__device__ __forceinline__ float rescale_weight(float m, float M) {
  return (m == -INFINITY) ? 0.0f : fast_exp2(m - M);
}

// Token range [s0, s1) of shard j of an L-token request split kvp ways:
// C = ceil(ceil(L / kvp) / 16) * 16, shard j = [j*C, min(L, (j+1)*C)).
__device__ __forceinline__ void shard_range(int64_t L, int kvp, int j, int64_t* s0, int64_t* s1) {
  int64_t per = (L + kvp - 1) / kvp;
  int64_t C = (per + 15) / 16 * 16;
  int64_t a = (int64_t)j * C;
  int64_t b = a + C;
  *s0 = a < L ? a : L;
  *s1 = b < L ? b : L;
}

// Cache layouts (kvd_layout of kvd.h).
enum CacheLayout : int { kContiguous = 0, kStriped = 1, kStaggered16 = 2, kPaged = 3 };

// What shard j of request b reads for KV head kvh on behalf of query token t
// of T: the slab (index of its [S_max, row] block in the cache tensor) and
// its token rows [s0, s1).
//  contiguous: cache [B,Hkv,S_max,.]; the split rule cuts [0, L).
//  striped / staggered16: cache [kvp,B,Hkv,S_max,.]; shard j holds its L_j
//  tokens at rows [0, L_j), L_j the number of positions i < L it owns
//  (i mod kvp == j, resp. (i div 16) mod kvp == j).
// Causal cut: query token t of a T-token turn sits at position L - T + t and
// sees positions below vis = L - T + 1 + t.  The positions a shard holds grow
// with its row, so what t sees of a shard is a prefix of its rows: the split
// rule's range cut at vis (contiguous, paged), or the owner count of the
// first vis positions (striped, staggered).  T = 1 sees the whole shard.
// Lengths are clamped so that no row outside the slab is ever read.
struct ShardSpan {
  int64_t slab, s0, s1;
};

__device__ __forceinline__ ShardSpan shard_span(int layout, int64_t L, int T, int t, int64_t S_max, int kvp,
                                                int B, int Hkv, int j, int b, int kvh) {
  ShardSpan sp;
  if (layout == kContiguous || layout == kPaged) {
    // (paged: S_max is the request capacity max_blocks * block_len; rows are
    // found through the block table, see phys_row)
    L = L < 0 ? 0 : (L > S_max ? S_max : L);
    const int64_t vis = L - (T - 1 - t);
    sp.slab = (int64_t)b * Hkv + kvh;
    shard_range(L, kvp, j, &sp.s0, &sp.s1);
    if (vis < sp.s1) sp.s1 = vis > sp.s0 ? vis : sp.s0;
    return sp;
  }
  const int64_t cap = S_max * kvp;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  int64_t vis = L - (T - 1 - t);
  vis = vis < 0 ? 0 : vis;
  int64_t Lj;
  if (layout == kStriped) {
    Lj = vis > j ? (vis - 1 - j) / kvp + 1 : 0;
  } else {
    const int64_t run = 16 * (int64_t)kvp;
    const int64_t full = vis / run;
    int64_t rem = vis - full * run - 16 * (int64_t)j;
    rem = rem < 0 ? 0 : (rem > 16 ? 16 : rem);
    Lj = 16 * full + rem;
  }
  sp.slab = ((int64_t)j * B + b) * Hkv + kvh;
  sp.s0 = 0;
  sp.s1 = Lj < S_max ? Lj : S_max;
  return sp;
}

// Workgroup id -> (work unit u, query token t) for a pass of U units with T
// query tokens each (see unit_token_blocks in kvd_internal.hpp for the grid).
// The T workgroups of one unit read the same cache rows.  Workgroups go to the
// 8 XCDs round-robin by id, so ids are laid out in groups of 8 units x T
// tokens, unit u and token t at id (u div 8) 8T + 8t + u mod 8: every token
// of a unit runs on the same XCD, where the rows one of them brings into that
// XCD's L2 serve the others, and they are dispatched back to back.  Returns
// false for the padding ids of a last, partial group of units.
__device__ __forceinline__ bool unit_token(int64_t id, int64_t U, int T, int64_t* u, int* t) {
  if (T == 1) {
    *u = id;
    *t = 0;
    return true;
  }
  const int64_t grp = id / (8 * (int64_t)T);
  const int r = (int)(id - grp * 8 * (int64_t)T);
  *t = r >> 3;
  *u = grp * 8 + (r & 7);
  return *u < U;
}

// Physical row (index into the cache tensor viewed as rows) of token t of
// request b, KV head kvh, for a shard with slab index `slab`.  Contiguous and
// sharded layouts: slab * S_max + t.  Paged: row t mod block_len of block
// block_table[b, t div block_len] (the id clamped into the pool); rows within
// one block are consecutive, so any 16-aligned run of 16 tokens (block_len is
// a power of two >= 16) is 16 consecutive physical rows.
template <class Args>
__device__ __forceinline__ int64_t phys_row(const Args& a, int b, int kvh, int64_t slab, int64_t t) {
  if (a.layout != kPaged) return slab * a.S_max + t;
  const int64_t lb = t >> a.log2_block;
  // The table is read-only while a kernel runs: reading it through the
  // constant address space lets a wave-uniform lookup be a scalar load, which
  // is waited for on its own counter instead of behind the cache loads in
  // flight.
  const __attribute__((address_space(4))) int32_t* table =
      (const __attribute__((address_space(4))) int32_t*)a.block_table;
  int64_t pb = table[(int64_t)b * a.max_blocks + lb];
  pb = pb < 0 ? 0 : (pb >= a.num_blocks ? a.num_blocks - 1 : pb);
  return ((pb * a.Hkv + kvh) << a.log2_block) + (t - (lb << a.log2_block));
}

// Where global position i lives: shard *j, row *r (contiguous: shard 0, row i).
__device__ __forceinline__ void token_home(int layout, int64_t i, int kvp, int* j, int64_t* r) {
  if (layout == kStriped) {
    *j = (int)(i % kvp);
    *r = i / kvp;
  } else if (layout == kStaggered16) {
    *j = (int)((i / 16) % kvp);
    *r = 16 * (i / (16 * (int64_t)kvp)) + i % 16;
  } else {
    *j = 0;
    *r = i;
  }
}

}  // namespace kvd
