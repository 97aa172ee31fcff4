// Split-KV partial attention for latent (MLA) heads on MFMA.
//
// Shape: 128 query heads share one cached latent row of 576 bf16 (512 latent +
// 64 rotary dims); V is the first 512 columns of the same row, so each cached
// byte is read from HBM once and serves both products:
//
//   S^T[token, head] = K_tile[token, 0:576] . Q[head, 0:576]
//   O^T[dv, head]   += K_tile[token, 0:512]^T . P^T[token, head]
//
// both on 32x32x16 MFMAs with fp32 accumulation: the logits on bf16, the PV
// product on fp16, with V converted from bf16 (exact below 2^16) and the
// weights P = 2^(logit - reference max + 7) rounded to fp16, the output
// normalized by the sum of those fp16 weights.  (The 32x32 MFMAs let the
// vector ALU work of a wave proceed under them, where 16x16 ones stall it for
// part of each instruction.)  The accumulator (256 AGPRs per wave) is never
// rescaled: see the pass structure below.
//
// Work split: one workgroup of 4 waves per (shard j, request b, KV head, query
// token; a single-token decode has one).  The shard is walked in 32-token
// tiles shared by all four waves.  Wave w computes the logits and weights of
// heads 32w .. 32w+31 (their Q, 144 VGPRs, stays in registers), the four
// waves exchange the fp16 weights through LDS, and wave w then accumulates
// value columns 128w .. 128w+127 of all 128 heads (256 AGPRs).  Per tile a
// wave reads the whole K tile for its logits and only its quarter of V.
//
// The tile loop is software-pipelined: the softmax of tile t - 1 runs in
// small pieces between the logits MFMAs of tile t (the vector ALU proceeds
// under a 32x32 MFMA), and once every wave's weights of tile t - 1 are in LDS
// the PV product of tile t - 1 follows, its V operands converted between its
// MFMAs one step ahead.
//
// Tiles travel HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging) into a
// ring of kBufs buffers, kAhead = 2 tiles ahead.  A buffer has two regions: the first
// 1024 bytes of each of the 32 rows (dims 0..511) at a stride of 65 16-byte
// slots, one row per load instruction, and the last 128 bytes (dims 512..575)
// at a stride of 9 slots, four rows per load instruction.  Every source
// address is a wave-uniform row pointer plus a fixed lane offset.  The odd
// row strides put the 16 rows a 16-lane group of a ds_read_b128 of K reads
// (one 16-byte slot each) on 16 different slots of the banks.  V^T operands
// come from ds_read_b64_tr_b16, whose 16-lane transpose turns four
// 16-column row segments into one column of 4 tokens per lane.
#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __fp16 h16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kHeads = 128;                 // query heads per KV head
constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDqk * 2;         // 1152
constexpr int kMainRowBytes = 1024;         // dims 0..511: one load instruction per row
constexpr int kTile = 32;
constexpr int kRowsPerWave = kTile / kWaves;
constexpr int kMainStride = 65;             // 16-byte slots per row, dims 0..511 (+1 pad)
constexpr int kTailStride = 9;              // 16-byte slots per row, dims 512..575 (+1 pad)
constexpr int kMainBytes = kTile * kMainStride * 16;   // 33280
constexpr int kTailBytes = kTile * kTailStride * 16;   // 4608
constexpr int kBufBytes = kMainBytes + kTailBytes;     // 37888
constexpr int kBufs = 4;
constexpr int kAhead = 2;                  // tiles issued ahead of the one whose logits run
constexpr int kLoads = kRowsPerWave + kRowsPerWave / 4;  // load instructions per wave per tile
constexpr int kSoftPieces = 18;            // softmax pieces per tile (two maxima, 16 weights)
constexpr int kKAhead = 4;                 // K operand reads in flight ahead of the logits MFMAs
constexpr int kPBytes = 8 * 64 * 16;        // fp16 weights of one tile, all 128 heads
// The fp16 weights are 2^kPOffset times exp2(logit - reference max): at most
// 2^(kPOffset + kHeadroom) = 2^15 < 65504 while no logit exceeds the
// reference by more than kHeadroom (log2 units), and 2^kPOffset at the max.
constexpr float kPOffset = 7.0f;
constexpr float kHeadroom = 8.0f;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4_t v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  f32x2_t f = {x, y};
  bf16x2_t h = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}

static_assert(2 * kLoads < 64, "vmcnt range");


// The logits MFMA with its accumulator in VGPRs.  The 256 AGPRs of a wave
// hold its PV accumulator, and the compiler gives every MFMA of a kernel the
// same (AGPR) form, so these are written out: acc (+)= K Q^T (first: acc =
// K Q^T).  The compiler does not see an MFMA here, so each block carries the
// hazard padding it would insert itself: 2 wait states between a vector-ALU
// write of an operand and the MFMA (s_nop 1), none between MFMAs chained on
// the same accumulator, and 12 before a vector-ALU read of the result
// (logit_mfma_drain, s_nop 15: 16).
__device__ __forceinline__ void logit_mfma(f32x16_t& acc, const uint4& k, const bf16x8_t& q, bool first) {
  const u32x4_t kv = u32x4_t{k.x, k.y, k.z, k.w};
  const u32x4_t qv = __builtin_bit_cast(u32x4_t, q);
  if (first)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(kv), "v"(qv));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(kv), "v"(qv));
}
// The drain names both accumulators as operands, so no read of them can be
// scheduled between the last MFMA and the padding.
__device__ __forceinline__ void logit_mfma_drain(f32x16_t& a0, f32x16_t& a1) {
  asm volatile("s_nop 15" : "+v"(a0), "+v"(a1));
}

// A wave-uniform pointer as scalar registers (the direct-to-LDS load takes
// its base address there).
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

// PAGED: rows are found through the block table (paged cache layout).
template <bool PAGED>
__global__ __launch_bounds__(kThreads) void mla_mfma_kernel(PartialArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int lane = threadIdx.x & 63;
  // wave index as a scalar, so everything derived from it stays wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;   // row / column of the 32x32 MFMA operands and results
  const int h2 = lane >> 5;    // which half of the 16-deep k block (operands) or 4-row groups (results)

  // unit (shard j, request b, KV head kvh) and query token qt
  int64_t unit;
  int qt;
  if (!unit_token(blockIdx.x, (int64_t)a.kvp * a.B * a.Hkv, a.T, &unit, &qt)) return;
  const int kvh = (int)(unit % a.Hkv);
  const int b = (int)(unit / a.Hkv % a.B);
  const int j = (int)(unit / ((int64_t)a.Hkv * a.B));
  const int64_t qrow0 = ((int64_t)b * a.T + qt) * a.Hq;                // q row of head h: qrow0 + h
  const int64_t orow0 = (((int64_t)j * a.B + b) * a.T + qt) * a.Hq;    // o_part / lse_part row

  const ShardSpan span = shard_span(a.layout, a.seq_lens[b], a.T, qt, a.S_max, a.kvp, a.B, a.Hkv, j, b, kvh);
  const int64_t s0 = span.s0, s1 = span.s1;
  const int64_t slab = span.slab;                  // cache block of this shard
  const int ntiles = (int)((s1 - s0 + kTile - 1) / kTile);
  const int64_t last = s1 - 1;

  // the cache viewed as rows; token t is row t of the slab (contiguous and
  // sharded layouts) or the row the block table gives (paged)
  const uint8_t* kdata = static_cast<const uint8_t*>(a.k) + (PAGED ? 0 : slab * a.S_max * kRowBytes);
  auto hrow = [&](int64_t t) -> int64_t {
    if constexpr (PAGED) {
      return phys_row(a, b, kvh, slab, t);
    } else {
      return t;
    }
  };
  const float c2 = a.scale_log2;
  const int head0 = kvh * kHeads + wave * 32;

  // Q^T operands of the 32x32x16 logits MFMAs: 36 chunks of 16 dims; lane l
  // holds head head0 + l % 32, dims 16 c + 8 (l / 32) .. +7 of chunk c.
  bf16x8_t qop[36];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (qrow0 + head0 + l32) * kDqk + 8 * h2;
#pragma unroll
    for (int c = 0; c < 36; ++c) {
      const uint4 v = *reinterpret_cast<const uint4*>(qrow + 16 * c);
      qop[c] = as_bf16x8(v.x, v.y, v.z, v.w);
    }
  }
  // Q is in registers before any cache load is issued, so the only vector
  // memory operations in flight inside the tile loop are the tile loads whose
  // counts the loop waits on explicitly.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)smem;
  // Rotary-dim loads: lane i < 36 fills slot i of a 4-row group, i.e. row
  // i / 9, chunk i % 9 of the row's last 8 chunks (the pad slot 8 repeats
  // chunk 7).
  // (Recomputed where used from an opaque copy of the lane index: a
  // per-lane constant held across the tile loop would be spilled, and its
  // reload would wait for every tile load in flight.)
  auto tail_lane = [&](int& row, uint32_t& off) {
    int l = lane;
    asm volatile("" : "+v"(l));
    row = l / 9;
    const int chunk = (l % 9) == 8 ? 7 : l % 9;
    off = (uint32_t)(kMainRowBytes + chunk * 16);
  };

  // Issue the direct-to-LDS loads of tile `tile` into buffer `buf`: this
  // wave's kRowsPerWave rows.  Rows past the shard end (last tile only) are
  // clamped to its last row.
  auto issue = [&](int tile, int buf) __attribute__((always_inline)) {
    const int64_t base = s0 + (int64_t)tile * kTile;
    const uint32_t bufaddr = lds0 + (uint32_t)(buf * kBufBytes);
    const int64_t g0 = base + kRowsPerWave * wave;   // this wave's first row (8-aligned)
    if (g0 + kRowsPerWave - 1 <= last) {
      // all 8 rows inside the shard; an aligned 8-row group is 8 consecutive
      // physical rows in every layout
      const uint8_t* src = uniform_ptr(kdata + hrow(g0) * kRowBytes);
#pragma unroll
      for (int k = 0; k < kRowsPerWave; ++k) {
        const int r = kRowsPerWave * wave + k;
        lds_dma16<true>(__builtin_amdgcn_readfirstlane(bufaddr + (uint32_t)(r * kMainStride * 16)),
                  src + k * kRowBytes, (uint32_t)(lane * 16));
      }
#pragma unroll
      for (int h = 0; h < kRowsPerWave / 4; ++h) {
        const int r0 = kRowsPerWave * wave + 4 * h;
        const uint32_t m0 =
            __builtin_amdgcn_readfirstlane(bufaddr + (uint32_t)(kMainBytes + r0 * kTailStride * 16));
        int tl_row;
        uint32_t tl_off;
        tail_lane(tl_row, tl_off);
        if (lane < 36) lds_dma16<true>(m0, src + 4 * h * kRowBytes, (uint32_t)(tl_row * kRowBytes) + tl_off);
      }
    } else {
      // last tile: rows clamped to the shard's last token
#pragma unroll
      for (int k = 0; k < kRowsPerWave; ++k) {
        const int r = kRowsPerWave * wave + k;
        int64_t row = base + r;
        row = row < last ? row : last;
        lds_dma16<true>(__builtin_amdgcn_readfirstlane(bufaddr + (uint32_t)(r * kMainStride * 16)),
                  uniform_ptr(kdata + hrow(row) * kRowBytes), (uint32_t)(lane * 16));
      }
#pragma unroll
      for (int h = 0; h < kRowsPerWave / 4; ++h) {
        const int r0 = kRowsPerWave * wave + 4 * h;
        const uint32_t m0 =
            __builtin_amdgcn_readfirstlane(bufaddr + (uint32_t)(kMainBytes + r0 * kTailStride * 16));
        // rows clamped per lane, relative to a clamped (in-shard) group base;
        // a 4-aligned group is 4 consecutive physical rows
        const int64_t row0 = base + r0;
        const int64_t rb = row0 < last ? row0 : last;
        int tl_row;
        uint32_t tl_off;
        tail_lane(tl_row, tl_off);
        int64_t row = row0 + tl_row;
        row = row < last ? row : last;
        const uint32_t off = (uint32_t)((row - rb) * kRowBytes) + tl_off;
        if (lane < 36) lds_dma16<true>(m0, uniform_ptr(kdata + hrow(rb) * kRowBytes), off);
      }
    }
  };

  // Per-lane LDS read offsets within a buffer.  K operand of chunk c: row
  // (token) l32, dims 16 c + 8 h2 .. +7: 16-byte slot 2 c + h2 of the row's
  // main region (c < 32) or 2 (c - 32) + h2 of its rotary region.
  const uint32_t k_main = (uint32_t)((l32 * kMainStride + h2) * 16);
  const uint32_t k_tail = (uint32_t)(kMainBytes + (l32 * kTailStride + h2) * 16);
  // V^T operand of 32 value columns and 16 tokens (step s of the tile): two
  // ds_read_b64_tr_b16, jj = 0, 1.  In 16-lane group G = lane / 16, lane
  // i = lane % 16 addresses row 16 s + 8 jj + 4 (G / 2) + i / 4, columns
  // 16 (G % 2) + 4 (i % 4) .. +3 of the block; the transpose hands lane i
  // column 16 (G % 2) + i = l32 of those four rows, which are k = 8 h2 +
  // 4 jj + 0..3 of the operand: token 16 s + 8 jj + 4 h2 + (k % 4).
  const int vg = lane >> 4, vi = lane & 15;
  const uint32_t v_off = (uint32_t)(((4 * (vg >> 1) + (vi >> 2)) * kMainStride) * 16 + 2 * (16 * (vg & 1) + 4 * (vi & 3)));
  // Result element e of a 32x32 block sits at row 8 (e / 4) + 4 h2 + e % 4,
  // column l32: logits of token 8 (e / 4) + 4 h2 + e % 4 for head l32, so
  // the PV step s takes elements 8 s .. 8 s + 7 as its P^T operand (tokens
  // 16 s + 8 jj + 4 h2 + i at k = 8 h2 + 4 jj + i, as in V^T).

  // This wave's share of the PV product: value columns 128 wave .. +127 of
  // all 128 heads; acc[d][H] holds O^T rows 128 wave + 32 d .. +31, heads
  // 32 H .. 32 H + 31.
  f32x16_t acc[4][4];
  // Softmax state of this wave's head head0 + l32 (both halves of the wave
  // hold the same): reference max (log2 domain), exact fp32 sum of the
  // weights and sum of the fp16 weights (over this lane's tokens).
  float m2 = -INFINITY, lsum = 0.f, lsum16 = 0.f;
  // The fp16 weights of all 128 heads for the current tile: head block H,
  // step s, lane l at ((2 H + s) 64 + l) 16 bytes (the P^T operand).
  const uint32_t p_lds = lds0 + (uint32_t)(kBufs * kBufBytes);
  float* const sum_lds = reinterpret_cast<float*>(smem + kBufs * kBufBytes);   // reused after the passes
  auto half_max = [](float v) {
    auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
  };
  auto half_sum = [](float v) {
    auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
  };

  // Pass structure.  The accumulating pass fixes each head's reference max
  // at its first tile and never rescales the accumulator; the fp16 weights
  // 2^(x c2 - m + kPOffset) stay below 2^15 while no tile exceeds its
  // reference by more than kHeadroom.  If one does, the workgroup reruns the
  // shard: a logits-only pass finds each head's exact max, then the
  // accumulating pass runs again with that max as the reference.  V enters
  // the PV product as fp16, exact for bf16 values below 2^16 in magnitude; if
  // a wave's columns hold a larger one, the shard is rerun with that wave's V
  // scaled by a power of two (vsc) that brings them into fp16's range, and
  // the wave's output scaled back.
  // Wait for tile `tile` (the loads of the tile issued after it may still be
  // in flight), meet the other waves (its loads have landed for all of them,
  // and all are done with the tile two back: its buffer and the weights in
  // LDS), issue the loads kAhead tiles on into that buffer; returns the
  // tile's valid rows (kTile or more except at the end).
  auto tile_ready = [&](int tile) __attribute__((always_inline)) {
    if (tile + 1 < ntiles) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoads));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    __builtin_amdgcn_s_barrier();
    if (tile + kAhead < ntiles) issue(tile + kAhead, (tile + kAhead) % kBufs);
    return (int)(s1 - (s0 + (int64_t)tile * kTile));
  };
  // Logits S^T[token, head] of the tile in buffer tb for its 32 tokens and
  // this wave's 32 heads: 36 chunks of 16 dims, K operands read kKAhead
  // chunks ahead (an LDS read under load takes longer than the 32-cycle
  // MFMA).  Element e: token 8 (e / 4) + 4 h2 + e % 4, head l32.  `between`
  // runs after MFMA step i (vector-ALU work that proceeds under the MFMAs);
  // the scheduling fences keep each step's work where it is written.
  auto tile_logits = [&](const uint8_t* tb, f32x16_t& sl, auto&& between) __attribute__((always_inline)) {
    auto kread = [&](int c) {
      const uint8_t* p = c < 32 ? tb + k_main + 32 * c : tb + k_tail + 32 * (c - 32);
      return *reinterpret_cast<const uint4*>(p);
    };
    // two accumulation chains (chunks 0..17 and 18..35), interleaved so that
    // no MFMA waits on the one just before it
    f32x16_t sl2;
    uint4 kq[kKAhead];
#pragma unroll
    for (int i = 0; i < kKAhead; ++i) kq[i] = kread((i & 1) * 18 + (i >> 1));
#pragma unroll
    for (int i = 0; i < 36; ++i) {
      const int c = (i & 1) * 18 + (i >> 1);     // chunk of step i
      const uint4 k0 = kq[i % kKAhead];
      if (i + kKAhead < 36) kq[i % kKAhead] = kread(((i + kKAhead) & 1) * 18 + ((i + kKAhead) >> 1));
      if (i & 1)
        logit_mfma(sl2, k0, qop[c], i == 1);
      else
        logit_mfma(sl, k0, qop[c], i == 0);
      between(i);
      __builtin_amdgcn_sched_barrier(0);
    }
    logit_mfma_drain(sl, sl2);
#pragma unroll
    for (int e = 0; e < 16; ++e) sl[e] += sl2[e];
  };
  auto no_work = [](int) {};
  // The tile's max logit of head l32 (tokens below nvalid), log2 domain.
  auto tile_max2 = [&](const f32x16_t& sl, int nvalid) {
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      tmax = fmaxf(tmax, (nvalid >= kTile || 8 * (e >> 2) + 4 * h2 + (e & 3) < nvalid) ? sl[e] : -INFINITY);
    return half_max(tmax) * c2;
  };

  bool max_only = false;
  float vsc = 1.0f;            // scale of this wave's V in the PV product
  bool vscaled = false;        // vsc != 1 (wave-uniform)
  float vmax = 0.0f;           // largest |V| this lane has converted
  for (;;) {
    // every pass starts from zero (so no pass carries the accumulator into
    // the next one)
    lsum = lsum16 = 0.f;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int H = 0; H < 4; ++H)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[d][H][e] = 0.f;
    int overflow = 0;
#pragma unroll
    for (int t = 0; t < kAhead; ++t)
      if (t < ntiles) issue(t, t);
    if (max_only) {
      // logits-only pass: each head's exact max over the shard
      for (int tile = 0; tile < ntiles; ++tile) {
        const int nvalid = tile_ready(tile);
        f32x16_t sl;
        tile_logits(smem + (tile % kBufs) * kBufBytes, sl, no_work);
        m2 = fmaxf(m2, tile_max2(sl, nvalid));
      }
      __syncthreads();           // every wave is past its last LDS read
      max_only = false;          // m2 now holds each head's exact max
      continue;
    }

    // ---- softmax weights of head l32 for a tile's logits sl (valid rows
    // nvalid): this lane's 16 tokens 8 (e / 4) + 4 h2 + e % 4, the other 16
    // in lane l ^ 32, in kSoftPieces pieces.  P = 2^(x c2 - m + kPOffset) (masked
    // logits give exp2(-inf) = 0), packed to fp16 toward zero and stored to
    // LDS; lsum takes the exact weights, lsum16 the fp16 ones the PV product
    // uses.
    float tmax = -INFINITY, pbase = 0.f, pe = 0.f;
    auto soft_piece = [&](int k, const f32x16_t& sl, int nvalid) __attribute__((always_inline)) {
      auto xv = [&](int e) {
        return (nvalid >= kTile || 8 * (e >> 2) + 4 * h2 + (e & 3) < nvalid) ? sl[e] : -INFINITY;
      };
      if (k == 0) {
        tmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) tmax = fmaxf(tmax, xv(e));
      } else if (k == 1) {
#pragma unroll
        for (int e = 8; e < 16; ++e) tmax = fmaxf(tmax, xv(e));
        const float tmax2 = half_max(tmax) * c2;
        if (m2 == -INFINITY) m2 = tmax2;      // first tile: acc is still zero
        overflow |= (tmax2 > m2 + kHeadroom);
        pbase = kPOffset - m2;
      } else if ((k & 1) == 0) {
        // weight of element 2 i
        const int i = (k - 2) >> 1;
        pe = fast_exp2(fmaf(xv(2 * i), c2, pbase));
        lsum += pe;
        asm volatile("" : "+v"(lsum), "+v"(pe));   // taken here, not deferred
      } else {
        // weight of element 2 i + 1; the pair to fp16, its sum, to LDS
        const int i = (k - 3) >> 1;
        const float p1 = fast_exp2(fmaf(xv(2 * i + 1), c2, pbase));
        lsum += p1;
        const h16x2_t pp = __builtin_amdgcn_cvt_pkrtz(pe, p1);
        lsum16 = __builtin_amdgcn_fdot2(pp, h16x2_t{(__fp16)1.0f, (__fp16)1.0f}, lsum16, false);
        asm volatile("" : "+v"(lsum), "+v"(lsum16));
        *(__attribute__((address_space(3))) uint32_t*)(uintptr_t)(
            p_lds + (uint32_t)(((2 * wave + (i >> 2)) * 64 + lane) * 16 + 4 * (i & 3))) =
            __builtin_bit_cast(uint32_t, pp);
      }
    };

    // ---- O^T += V^T P^T for the tile in buffer buf: this wave's 4 blocks of
    // 32 value columns against the weights of all 4 head blocks, two 16-token
    // steps each; V^T operands converted to fp16 one step ahead of their MFMAs
    auto tile_pv = [&](int buf) __attribute__((always_inline)) {
      const uint8_t* tb = smem + buf * kBufBytes;
      if (vscaled) {
        // rerun with this wave's V scaled by vsc (a V element beyond fp16):
        // scale its 128 columns of the tile in LDS, which only this wave
        // reads from here on (every logits read of the tile is done), exactly
        // (a power of two; bf16 keeps fp32's exponent range)
        // 16-byte chunk 64 i + lane: row 4 i + lane / 16, column chunk lane % 16
        lds_u32x4* const q0 = (lds_u32x4*)(uintptr_t)(lds0 + (uint32_t)(buf * kBufBytes) +
                                                      (uint32_t)((lane >> 4) * kMainStride * 16 + 256 * wave + (lane & 15) * 16));
#pragma unroll 1
        for (int i = 0; i < 8; ++i) {      // one chunk at a time: a rare path, kept light on registers
          lds_u32x4* q16 = q0 + i * 4 * kMainStride;
          u32x4_t w = *q16;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float lo = __uint_as_float(w[k] << 16) * vsc, hi = __uint_as_float(w[k] & 0xFFFF0000u) * vsc;
            w[k] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
          }
          *q16 = w;
        }
      }
      const uint8_t* vbase = tb + v_off + 2 * 128 * wave;
      auto vraw = [&](int d, int st) {
        const uint8_t* p = vbase + 2 * 32 * d + 16 * st * kMainStride * 16;
        const uint2 w0 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p));
        const uint2 w1 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                      (lds_s16x4_t*)(p + 8 * kMainStride * 16)));
        return u32x4_t{w0.x, w0.y, w1.x, w1.y};
      };
      // bf16 -> fp16 of one V^T operand dword (two values), tracking |V|
      auto vconv = [&](uint32_t w) {
        const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xFFFF0000u);
        vmax = fmaxf(fmaxf(vmax, fabsf(lo)), fabsf(hi));
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
      };
      u32x4_t pw[4][2];
#pragma unroll
      for (int H = 0; H < 4; ++H)
#pragma unroll
        for (int st = 0; st < 2; ++st)
          pw[H][st] = *(const lds_u32x4*)(uintptr_t)(p_lds + (uint32_t)(((2 * H + st) * 64 + lane) * 16));
      // step ds = (d, st): the raw V^T operand is read two steps ahead and
      // converted one step ahead, between the four MFMAs of the step before
      u32x4_t vr1 = vraw(0, 1), va;
      {
        const u32x4_t vr0 = vraw(0, 0);
#pragma unroll
        for (int k = 0; k < 4; ++k) va[k] = vconv(vr0[k]);
      }
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) {
        const int d = ds >> 1, st = ds & 1;
        u32x4_t vr2 = vr1;
        if (ds + 2 < 8) vr2 = vraw((ds + 2) >> 1, (ds + 2) & 1);
        u32x4_t vn = va;
#pragma unroll
        for (int H = 0; H < 4; ++H) {
          acc[d][H] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, va),
                                                             __builtin_bit_cast(f16x8_t, pw[H][st]), acc[d][H], 0, 0, 0);
          if (ds + 1 < 8) vn[H] = vconv(vr1[H]);
        }
        va = vn;
        vr1 = vr2;
#pragma unroll
        for (int H = 0; H < 4; ++H) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // then a conversion's vector-ALU work
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Software pipeline over the tiles: the logits of tile t run with the
    // softmax of tile t - 1 in their shadow; then, once every wave's weights
    // are in LDS, the PV product of tile t - 1.  Only the last tile can be
    // partial, so every softmax inside the loop is over a full tile.
    if (ntiles > 0) {
      f32x16_t sp;                              // logits of the previous tile
      tile_ready(0);
      tile_logits(smem, sp, no_work);
      for (int tile = 1; tile < ntiles; ++tile) {
        tile_ready(tile);
        f32x16_t sl;
        tile_logits(smem + (tile % kBufs) * kBufBytes, sl, [&](int i) {
          if ((i & 1) == 0) soft_piece(i >> 1, sp, kTile);
        });
        __syncthreads();                        // every wave's weights are in LDS
        tile_pv((tile - 1) % kBufs);
        sp = sl;
      }
      // the last tile: its softmax, then its PV product
      __syncthreads();                          // every wave is past the previous weights
      const int nlast = (int)(s1 - (s0 + (int64_t)(ntiles - 1) * kTile));
#pragma unroll
      for (int k = 0; k < kSoftPieces; ++k) soft_piece(k, sp, nlast);
      __syncthreads();
      tile_pv((ntiles - 1) % kBufs);
    }
    // a V element of this wave's columns beyond fp16 (on the unscaled pass)
    if (!vscaled && __any(vmax >= 65520.0f)) overflow |= 2;
    // every wave is past its last LDS read before the buffers are refilled
    // (bit 0: a logit beyond the headroom; bit 1: a V element beyond fp16)
    const int flags = __syncthreads_or(overflow);
    if (!flags) break;
    if (overflow & 2) {
      // V x 2^-k, with the wave's largest |V| below 2^(14 + k), fits fp16
      // (an infinite V element stays infinite: k = 0)
      const float wmax = rows4_max(row16_max(vmax));
      const int k = __builtin_amdgcn_readfirstlane(isinf(wmax) ? 0 : min(120, (int)ceilf(fast_log2(wmax)) - 14));
      vsc = __uint_as_float((uint32_t)(127 - k) << 23);
      vscaled = k > 0;
    }
    if (flags & 1) {
      max_only = true;
      m2 = -INFINITY;
    }                            // else: the same reference max again
  }

  // ---- lse of this wave's 32 heads; the fp16 weight sums of all 128 heads
  // through LDS (the buffers are idle after the final barrier above)
  {
    const float lt = half_sum(lsum);
    const float l16 = half_sum(lsum16);
    const bool empty = (m2 == -INFINITY);
    const int h = wave * 32 + l32;
    if (h2 == 0) {
      a.lse_part[orow0 + kvh * kHeads + h] = empty ? -INFINITY : (m2 - kPOffset + fast_log2(lt)) * kLn2;
      sum_lds[h] = empty ? 0.0f : l16;
    }
  }
  __syncthreads();
  // ---- write this wave's 128 value columns of every head, normalized:
  // element e of acc[d][H] is column 128 wave + 32 d + 8 (e / 4) + 4 h2 + e % 4
#pragma unroll
  for (int H = 0; H < 4; ++H) {
    const int h = 32 * H + l32;
    const float l16 = sum_lds[h];
    const float inv = l16 > 0.0f ? 1.0f / (l16 * vsc) : 0.0f;
    float* orow = a.o_part + (orow0 + kvh * kHeads + h) * kDv + 128 * wave + 4 * h2;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(orow + 32 * d + 8 * j) =
            make_float4(acc[d][H][4 * j] * inv, acc[d][H][4 * j + 1] * inv, acc[d][H][4 * j + 2] * inv,
                        acc[d][H][4 * j + 3] * inv);
  }
}

constexpr size_t kSmemBytes = (size_t)kBufs * kBufBytes + kPBytes;
static_assert(kSmemBytes <= 160 * 1024, "LDS budget");
static_assert((kTile - 1) * kMainStride * 16 + kMainRowBytes <= kMainBytes, "row loads stay in the main region");
static_assert(kMainBytes + (kTile - 4) * kTailStride * 16 + 4 * kTailStride * 16 <= kBufBytes,
              "rotary loads stay in the buffer");

}  // namespace

bool mla_mfma_supports(const PartialArgs& a) {
  return a.q_bf16 && a.kv_format == kBF16 && a.v_aliases_k && a.Dqk == kDqk && a.Dv == kDv &&
         a.Hq / a.Hkv == kHeads;
}

hipError_t launch_partial_mla_mfma(const PartialArgs& a, hipStream_t stream) {
  // more than 64 KB of dynamic LDS: raise both instances' limit once (the
  // initialization of a local static is thread-safe)
  static const hipError_t attr = [] {
    for (const void* fn : {reinterpret_cast<const void*>(mla_mfma_kernel<false>),
                           reinterpret_cast<const void*>(mla_mfma_kernel<true>)}) {
      const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmemBytes);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }();
  if (attr != hipSuccess) return attr;
  const int64_t blocks = unit_token_blocks((int64_t)a.kvp * a.B * a.Hkv, a.T);
  if (a.layout == kPaged)
    hipLaunchKernelGGL(mla_mfma_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), kSmemBytes, stream, a);
  else
    hipLaunchKernelGGL(mla_mfma_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), kSmemBytes, stream, a);
  return hipGetLastError();
}

}  // namespace kvd
