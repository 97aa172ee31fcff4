// Split-KV partial attention of three or four query tokens of one request
// (a pass-Q turn) for a group of 16 query heads on an fp8 (E4M3) cache, on
// 32x32x16 MFMAs: one wave per (shard, request, KV head) decodes each
// 32-token tile once and serves all the tokens from it.
//
// The matrix-core columns are (query token, head) pairs: columns 0..31 of
// block nb are tokens 2 nb and 2 nb + 1 (16 heads each), so
//
//   S^T[token, (i, h)] = K_tile[token, :] . Q[i, h, :]        (bf16 MFMA, K decoded exactly)
//   O^T[dv, (i, h)]   += V_tile[:, dv]^T . P^T[token, (i, h)]  (fp16 MFMA, V decoded exactly)
//
// with P = 2^(s - m + 7) rounded toward zero to fp16 and the output
// normalized by the sum of those fp16 weights (the log-sum-exp takes the
// exact fp32 sum).  The running max of each column moves only when a tile's
// max exceeds it by more than 2^8, as in the single-token kernel.  Causality:
// token i sees the rows below its own cut (shard_span of token i).
//
// Tiles travel HBM -> LDS with global_load_lds_dwordx4 into a ring of kSlots
// slots per wave (K, then V, 32 rows of 128 bytes each).  Slots are unpadded:
// 16-byte chunk c of row r sits at chunk c ^ g(r) (K) or c ^ f(r) (V) of its
// row, permuted by the loading lanes, so that the 16 lanes of a K read and
// the 32 lanes of a V read fall on distinct banks.  K operands are read with
// ds_read_b128 (lane: token l32, dims 64 h2 .. 64 h2 + 63 in the k order the
// query operands use); V operands with ds_read_b64_tr_b8, whose 16-lane
// transpose hands each lane one value column of 8 tokens: the k order of the
// P^T operand, so no byte shuffles are needed.
#include <type_traits>

#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __fp16 h16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;

constexpr int kWaves = 4;                 // independent waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kD = 128;
constexpr int kG = 16;                    // query heads per KV head
constexpr int kTile = 32;
constexpr int kRow = 128;                 // bytes of an fp8 row
constexpr int kHalf = kTile * kRow;       // K or V part of a slot
constexpr int kSlotBytes = 2 * kHalf;
constexpr int kSlots = 4;
constexpr int kWaveBytes = kSlots * kSlotBytes;
constexpr int kDma = kHalf / 1024;        // load instructions per part (8 rows each)
constexpr int kLoads = 2 * kDma;          // per tile
constexpr float kLazyMax = 8.0f;
constexpr float kPOffset = 7.0f;

// Chunk permutations (16-byte chunks, 8 to a row): K reads take one chunk of
// 16 consecutive rows, V reads two chunks of 8 rows {0..3, 8..11} + 4 h2 of a
// 16-row step; g and f give those rows' chunks distinct banks.
__device__ __forceinline__ constexpr int gk(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ constexpr int fv(int r) { return 2 * (((r >> 1) & 1) | ((r >> 2) & 2)); }

__device__ __forceinline__ bf16x8_t bf16_from_fp8(uint32_t w0, uint32_t w1) {
  u32x4_t v = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true))};
  return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ f16x8_t f16_from_fp8(uint32_t w0, uint32_t w1) {
  u32x4_t v = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true))};
  return __builtin_bit_cast(f16x8_t, v);
}

// The logits MFMA with the query operand in AGPRs (so the 128 accumulator
// values of the PV product can stay in VGPRs): acc (+)= K Q^T.  Written out,
// since the compiler would take the operands of its own MFMAs from VGPRs, so
// each carries the hazard padding the compiler would insert: 2 wait states
// after a vector-ALU write of the K operand (s_nop 1), none between chained
// MFMAs, and 16 before a vector-ALU read of the result (logit_drain).
__device__ __forceinline__ void logit_mfma(f32x16_t& acc, const bf16x8_t& k, const u32x4_t& q, bool first) {
  const u32x4_t kv = __builtin_bit_cast(u32x4_t, k);
  if (first)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(kv), "a"(q));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(kv), "a"(q));
}
// The drain names the accumulator as an operand, so no read of it can be
// scheduled between the last MFMA and the padding.
__device__ __forceinline__ void logit_drain(f32x16_t& acc) { asm volatile("s_nop 15" : "+v"(acc)); }
__device__ __forceinline__ void logit_drain(f32x16_t& a0, f32x16_t& a1) { asm volatile("s_nop 15" : "+v"(a0), "+v"(a1)); }

// One direct-to-LDS 16-byte load per lane from sbase + voff + OFF into LDS
// address m0 + OFF + 16 lane: the instruction's immediate offset applies to
// both addresses.  Non-temporal.  M0 belongs to the compiler: saved and
// restored around the load.
template <int OFF>
__device__ __forceinline__ void dma16(uint32_t m0, const uint8_t* sbase, uint32_t voff) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3 offset:%4 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "s"(m0), "v"(voff), "s"(sbase), "n"(OFF)
      : "memory");
}

// A wave-uniform pointer as a scalar value (the load instructions take their
// base address from SGPRs; the compiler may have computed it in VGPRs).
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

// PAGED: rows are found through the block table (paged cache layout).
// NB: column blocks (tokens 0 .. 2 NB - 1); the launcher uses NB = 2 (three
// or four tokens; the columns of a fourth token past T are computed on a
// zero query and not written).
template <bool PAGED, int NB>
__global__ __launch_bounds__(kThreads) void gqa_fp8_tokens32_kernel(PartialArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int h2 = lane >> 5;

  // unit (shard j, request b, KV head kvh), one per wave
  const int64_t unit = (int64_t)blockIdx.x * kWaves + wave;
  if (unit >= (int64_t)a.kvp * a.B * a.Hkv) return;   // the whole wave: no barrier follows
  const int kvh = (int)(unit % a.Hkv);
  const int b = (int)(unit / a.Hkv % a.B);
  const int j = (int)(unit / ((int64_t)a.Hkv * a.B));
  const int T = a.T;

  // Rows of the shard: [s0, s1); token i sees [s0, s1t[i]).
  const int64_t L = a.seq_lens[b];
  const ShardSpan span = shard_span(a.layout, L, T, T - 1, a.S_max, a.kvp, a.B, a.Hkv, j, b, kvh);
  const int64_t s0 = span.s0, s1 = span.s1;
  int64_t s1t[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    s1t[i] = i >= T ? s0 : shard_span(a.layout, L, T, i, a.S_max, a.kvp, a.B, a.Hkv, j, b, kvh).s1;
  const int64_t slab = span.slab;
  const int64_t last = s1 - 1;
  const int ntiles = (int)((s1 - s0 + kTile - 1) / kTile);
  const int64_t bh = (int64_t)b * a.Hkv + kvh;

  const uint8_t* kdata = static_cast<const uint8_t*>(a.k) + (PAGED ? 0 : slab * a.S_max * kRow);
  const uint8_t* vdata = static_cast<const uint8_t*>(a.v) + (PAGED ? 0 : slab * a.S_max * kRow);
  auto hrow = [&](int64_t t) -> int64_t {
    if constexpr (PAGED) {
      return phys_row(a, b, kvh, slab, t);
    } else {
      return t;
    }
  };
  const float kscale = static_cast<const float*>(a.k_scale)[bh];
  const float vscale = static_cast<const float*>(a.v_scale)[bh];
  // raw logit -> log2 domain; a negative K scale is carried by the query
  // operands' sign, so c2 >= 0
  const float c2 = a.scale_log2 * fabsf(kscale);
  const uint32_t qsign = kscale < 0.0f ? 0x80008000u : 0u;

  // Q^T operands: block nb, k-step c: lane (n = l32, h2) holds token
  // 2 nb + n / 16, head n % 16, dims 64 h2 + 8 c .. +7 (zero for tokens past
  // T).
  u32x4_t qop[NB][8];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int i = 2 * nb + (l32 >> 4);
    const bool ok = i < T;
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + (((int64_t)b * T + (ok ? i : 0)) * a.Hq + kvh * kG + (l32 & 15)) * kD + 64 * h2;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint4 v = *reinterpret_cast<const uint4*>(qrow + 8 * c);
      if (!ok) v = make_uint4(0u, 0u, 0u, 0u);
      qop[nb][c] = u32x4_t{v.x ^ qsign, v.y ^ qsign, v.z ^ qsign, v.w ^ qsign};
    }
  }
  // Q is in registers before any cache load is issued, so the only vector
  // memory operations in flight in the tile loop are the tile loads.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  const uint32_t ring = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)smem +
                        (uint32_t)(wave * kWaveBytes);
  // Loads: instruction q of a part fills rows 8 q .. 8 q + 7; lane i writes
  // slot byte 16 i, i.e. row 8 q + i / 8, chunk slot i % 8, so it fetches
  // chunk (i % 8) ^ perm(row) of that row.
  auto lane_src = [&](int q, bool isv) -> uint32_t {
    const int r = 8 * q + (lane >> 3);
    const int p = isv ? fv(r) : gk(r);
    return (uint32_t)((lane >> 3) * kRow + 16 * ((lane & 7) ^ p));
  };
  const uint32_t lk[kDma] = {lane_src(0, false), lane_src(1, false), lane_src(2, false), lane_src(3, false)};
  const uint32_t lv[2] = {lane_src(0, true), lane_src(1, true)};
  auto issue = [&](int tile, int slot) {
    const int64_t base = s0 + (int64_t)tile * kTile;
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(ring + (uint32_t)(slot * kSlotBytes));
    if (base + kTile - 1 <= last) {
      // a whole tile: 32 consecutive physical rows (paged: two runs of 16)
      if constexpr (!PAGED) {
        const uint8_t* kp = uniform_ptr(kdata + base * kRow);
        const uint8_t* vp = uniform_ptr(vdata + base * kRow);
        dma16<0>(m0, kp, lk[0]);
        dma16<1024>(m0, kp, lk[1]);
        dma16<2048>(m0, kp, lk[2]);
        dma16<3072>(m0, kp, lk[3]);
        dma16<0>(m0 + kHalf, vp, lv[0]);
        dma16<1024>(m0 + kHalf, vp, lv[1]);
        dma16<2048>(m0 + kHalf, vp, lv[0]);
        dma16<3072>(m0 + kHalf, vp, lv[1]);
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int64_t pr = hrow(base + 16 * u);
          const uint8_t* kp = uniform_ptr(kdata + pr * kRow);
          const uint8_t* vp = uniform_ptr(vdata + pr * kRow);
          dma16<0>(m0 + (uint32_t)(2048 * u), kp, lk[2 * u]);
          dma16<1024>(m0 + (uint32_t)(2048 * u), kp, lk[2 * u + 1]);
          dma16<0>(m0 + (uint32_t)(kHalf + 2048 * u), vp, lv[0]);
          dma16<1024>(m0 + (uint32_t)(kHalf + 2048 * u), vp, lv[1]);
        }
      }
    } else {
      // the last tile: rows past the shard end clamped to its last row, lane
      // by lane
#pragma unroll
      for (int q = 0; q < kDma; ++q) {
        const uint32_t mk = m0 + (uint32_t)(q * 1024), mv = mk + (uint32_t)kHalf;
        int64_t row = base + 8 * q + (lane >> 3);
        row = row < last ? row : last;
        const int64_t pr = hrow(row);
        const uint32_t off = lk[q] - (uint32_t)((lane >> 3) * kRow);
        const uint32_t offv = lv[q & 1] - (uint32_t)((lane >> 3) * kRow);
        lds_dma16_at(mk, kdata + pr * kRow + off);
        lds_dma16_at(mv, vdata + pr * kRow + offv);
      }
    }
  };

  // K reads: chunk 4 h2 + c2 (dims 64 h2 + 16 c2 .. +15) of row l32
  const uint32_t k_rd = (uint32_t)(l32 * kRow);
  const int k_p = gk(l32);
  // V reads (block mblk, step st): lane (G = lane / 16, i = lane % 16) reads
  // row 16 st + 8 (i / 8) + 4 h2 + (i / 2) % 4, bytes 8 (i % 2) .. +7 of
  // chunk 2 mblk + G % 2; the transpose gives lane i column 16 (G % 2) + i
  // = l32 of the 8 rows in that order: tokens 16 st + 8 (k / 4) + 4 h2 +
  // k % 4 for k = 0..7, the P^T operand's.
  const int v_row = 8 * ((lane & 15) >> 3) + 4 * h2 + ((lane >> 1) & 3);
  const int v_fp = fv(v_row);
  const int v_g = (lane >> 4) & 1;
  const uint32_t v_rd = (uint32_t)(kHalf + v_row * kRow + 8 * (lane & 1));

  f32x16_t acc[4][NB];   // O^T: value columns 32 mblk .. +31, column block nb
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[m][nb][e] = 0.f;
  float m2[2] = {-INFINITY, -INFINITY};   // running max of column l32 (log2)
  float lsum[2] = {0.f, 0.f};             // fp32 weights, this lane's rows
  float lsum16[2] = {0.f, 0.f};           // fp16 weights, this lane's rows

  auto half_max = [](float v) {
    auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
  };
  auto half_sum = [](float v) {
    auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
  };

  // Softmax weights of column block nb on one tile, in steps that can be
  // spread over MFMAs: soft_begin (mask, tile max, running-max move), then
  // soft_pair(e2), e2 = 0..7: the fp16 weights of elements 2 e2, 2 e2 + 1
  // of lane (n, h2), tokens 8 (e / 4) + 4 h2 + e % 4 of the tile for column
  // n.  MASK: rows at or past the column's token cut get weight 0.
  auto soft_begin = [&](auto mask_tag, int nb, f32x16_t& x, const int (&nv)[4]) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if constexpr (MASK) {
      // (arithmetic select: an indexed pick would put nv in scratch)
      const int n0 = nv[2 * nb], n1 = nv[2 * nb + 1];
      const int lim = n0 + ((l32 >> 4) & 1) * (n1 - n0) - 4 * h2;
#pragma unroll
      for (int e = 0; e < 16; ++e) x[e] = (8 * (e >> 2) + (e & 3)) < lim ? x[e] : -INFINITY;
    }
    float tmax = x[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) tmax = fmaxf(tmax, x[e]);
    const float tmax2 = half_max(tmax) * c2;   // both halves of column n agree
    if (__any(tmax2 > m2[nb] + kLazyMax)) {
      // move the running max (only where it rises by more than 2^8: the
      // stale max is exact algebra and keeps the weights below 2^15);
      // columns whose max does not move keep their state (one still at
      // -inf, all its rows masked so far, would otherwise get exp2(NaN))
      const bool mv = tmax2 > m2[nb] + kLazyMax;
      const float mn = mv ? tmax2 : m2[nb];
      const float al = mv ? fast_exp2(m2[nb] - mn) : 1.0f;
      lsum[nb] *= al;
      lsum16[nb] *= al;
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[m][nb] *= al;
      m2[nb] = mn;
    }
  };
  auto soft_pair = [&](auto mask_tag, int nb, const f32x16_t& x, int e2, uint32_t& ph) {
    constexpr bool MASK = decltype(mask_tag)::value;
    float p0 = fast_exp2(fmaf(x[2 * e2], c2, kPOffset - m2[nb]));
    float p1 = fast_exp2(fmaf(x[2 * e2 + 1], c2, kPOffset - m2[nb]));
    if constexpr (MASK) {
      p0 = x[2 * e2] == -INFINITY ? 0.0f : p0;
      p1 = x[2 * e2 + 1] == -INFINITY ? 0.0f : p1;
    }
    lsum[nb] += p0 + p1;
    const h16x2_t pp = __builtin_amdgcn_cvt_pkrtz(p0, p1);
    lsum16[nb] = __builtin_amdgcn_fdot2(pp, h16x2_t{(__fp16)1.0f, (__fp16)1.0f}, lsum16[nb], false);
    ph = __builtin_bit_cast(uint32_t, pp);
  };

  // One tile from the slot at LDS address sb: nv[i] valid rows for token i;
  // NB column blocks (tokens 0..2 NB - 1).  Both blocks' logits share the
  // decoded K; then block 0's PV product runs with block 1's softmax in
  // between its MFMAs, and block 1's PV product last (V decoded again).
  auto compute = [&](auto mask_tag, uint32_t sb, const int (&nv)[4]) {
    // the K reads of the tile up front, the V reads once the logits are issued
    u32x4_t kw[4];
#pragma unroll
    for (int c2i = 0; c2i < 4; ++c2i)
      kw[c2i] = *(const lds_u32x4*)(uintptr_t)(sb + k_rd + (uint32_t)(16 * ((4 * h2 + c2i) ^ k_p)));
    // ---- logits of the column blocks, K decoded once
    f32x16_t sl[NB];
#pragma unroll
    for (int c2i = 0; c2i < 4; ++c2i) {
      const bf16x8_t k0 = bf16_from_fp8(kw[c2i][0], kw[c2i][1]);
      const bf16x8_t k1 = bf16_from_fp8(kw[c2i][2], kw[c2i][3]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) logit_mfma(sl[nb], k0, qop[nb][2 * c2i], c2i == 0);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) logit_mfma(sl[nb], k1, qop[nb][2 * c2i + 1], false);
    }
    i32x2_t vw[2][4];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        vw[st][m] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(uintptr_t)(
            sb + v_rd + (uint32_t)(16 * st * kRow) + (uint32_t)(16 * ((2 * m + v_g) ^ v_fp))));
    if constexpr (NB == 2)
      logit_drain(sl[0], sl[NB - 1]);
    else
      logit_drain(sl[0]);
    // ---- block 0: weights, then its PV product with block 1's weights
    // computed in between
    u32x4_t pw0[2], pw1[2];
    {
      uint32_t ph[8];
      soft_begin(mask_tag, 0, sl[0], nv);
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) soft_pair(mask_tag, 0, sl[0], e2, ph[e2]);
      pw0[0] = u32x4_t{ph[0], ph[1], ph[2], ph[3]};
      pw0[1] = u32x4_t{ph[4], ph[5], ph[6], ph[7]};
    }
    uint32_t ph1[8];
    if constexpr (NB == 2) soft_begin(mask_tag, 1, sl[NB - 1], nv);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f16x8_t vop = f16_from_fp8((uint32_t)vw[st][m][0], (uint32_t)vw[st][m][1]);
        acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, __builtin_bit_cast(f16x8_t, pw0[st]), acc[m][0], 0, 0, 0);
        if constexpr (NB == 2) soft_pair(mask_tag, 1, sl[NB - 1], 4 * st + m, ph1[4 * st + m]);
      }
    }
    if constexpr (NB == 2) {
      pw1[0] = u32x4_t{ph1[0], ph1[1], ph1[2], ph1[3]};
      pw1[1] = u32x4_t{ph1[4], ph1[5], ph1[6], ph1[7]};
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f16x8_t vop = f16_from_fp8((uint32_t)vw[st][m][0], (uint32_t)vw[st][m][1]);
          acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, __builtin_bit_cast(f16x8_t, pw1[st]), acc[m][1], 0, 0, 0);
        }
    }
  };

  // ---- the tile ring: tiles kSlots - 1 ahead
#pragma unroll
  for (int t = 0; t < kSlots - 1; ++t)
    if (t < ntiles) issue(t, t);
  // Tiles below nclean are whole for every token; the rest (the causal
  // tail and a partial last tile) are masked.
  int nclean = ntiles;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < T) {
      const int f = (int)((s1t[i] - s0) / kTile);
      nclean = f < nclean ? f : nclean;
    }
  auto step = [&](int tile, auto mask_tag) {
    const int ahead = ntiles - 1 - tile;   // tiles issued after this one (at most kSlots - 2)
    if (ahead >= 2) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLoads));
    } else if (ahead == 1) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoads));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    asm volatile("" ::: "memory");
    if (tile + kSlots - 1 < ntiles) issue(tile + kSlots - 1, (tile + kSlots - 1) % kSlots);
    const int64_t base = s0 + (int64_t)tile * kTile;
    int nv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t n = s1t[i] - base;
      nv[i] = n < 0 ? 0 : (n > kTile ? kTile : (int)n);
    }
    compute(mask_tag, ring + (uint32_t)((tile % kSlots) * kSlotBytes), nv);
  };
  for (int tile = 0; tile < nclean; ++tile) step(tile, std::false_type{});
  for (int tile = nclean; tile < ntiles; ++tile) step(tile, std::true_type{});

  // ---- normalized partials and natural-log lse of each token and head
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int i = 2 * nb + (l32 >> 4);
    const float lw = half_sum(lsum[nb]);
    const float l16 = half_sum(lsum16[nb]);
    if (i >= T) continue;
    const bool empty = m2[nb] == -INFINITY || !(l16 > 0.0f);
    const float inv = empty ? 0.0f : vscale / l16;
    const int64_t orow = (((int64_t)j * a.B + b) * T + i) * a.Hq + kvh * kG + (l32 & 15);
    float* dst = a.o_part + orow * kD + 4 * h2;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *reinterpret_cast<float4*>(dst + 32 * m + 8 * k) =
            make_float4(acc[m][nb][4 * k] * inv, acc[m][nb][4 * k + 1] * inv, acc[m][nb][4 * k + 2] * inv,
                        acc[m][nb][4 * k + 3] * inv);
    if (h2 == 0) a.lse_part[orow] = empty ? -INFINITY : (m2[nb] - kPOffset + fast_log2(lw)) * kLn2;
  }
}

static_assert(kWaves * kWaveBytes <= 160 * 1024, "LDS ring budget");
static_assert(2 * kLoads < 64, "vmcnt range");

}  // namespace

bool gqa_tokens32_supports(const PartialArgs& a) {
  return a.q_bf16 && !a.v_aliases_k && a.kv_format == kFP8 && a.Dqk == kD && a.Dv == kD &&
         a.Hq == kG * a.Hkv && a.T >= 3 && a.T <= 4;
}

hipError_t launch_gqa_tokens32(const PartialArgs& a, hipStream_t stream) {
  constexpr size_t kLds = (size_t)kWaves * kWaveBytes;
  static const hipError_t attr = [] {
    for (const void* fn : {reinterpret_cast<const void*>(gqa_fp8_tokens32_kernel<false, 2>),
                           reinterpret_cast<const void*>(gqa_fp8_tokens32_kernel<true, 2>)}) {
      const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }();
  if (attr != hipSuccess) return attr;
  const int64_t units = (int64_t)a.kvp * a.B * a.Hkv;
  const dim3 grid((unsigned)((units + kWaves - 1) / kWaves)), block(kThreads);
  if (!gqa_tokens32_supports(a)) return hipErrorInvalidValue;
  if (a.layout == kPaged)
    hipLaunchKernelGGL((gqa_fp8_tokens32_kernel<true, 2>), grid, block, kLds, stream, a);
  else
    hipLaunchKernelGGL((gqa_fp8_tokens32_kernel<false, 2>), grid, block, kLds, stream, a);
  return hipGetLastError();
}

}  // namespace kvd
