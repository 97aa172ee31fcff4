// Split-KV partial attention for latent (MLA) heads on MFMA.
//
// Shape: 128 query heads share one cached latent row of 576 bf16 (512 latent +
// 64 rotary dims); V is the first 512 columns of the same row, so each cached
// byte is read from HBM once and serves both products:
//
//   S^T[token, head] = K_tile[token, 0:576] . Q[head, 0:576]   (18 MFMAs / 16x16 block)
//   O^T[dv, head]   += K_tile[token, 0:512]^T . P^T[token, head]
//
// both on v_mfma_f32_16x16x32_bf16 with fp32 accumulation; P enters the PV
// product as a bf16 hi + lo pair (two MFMAs), as in the GQA kernel.  The
// accumulator (256 AGPRs per wave) is never rescaled: see the pass structure
// below.
//
// Work split: one workgroup of 4 waves per (shard j, request b, KV head, query
// token; a single-token decode has one).  The
// shard is walked in 32-token tiles shared by all four waves; wave w owns heads
// 32w .. 32w+31, keeping their Q (144 VGPRs) and their O^T accumulator (32 heads
// x 512 dv, 256 AGPRs) in registers for the whole shard; LDS traffic per
// cached token is 4 x (1152 + 1024) bytes.
//
// Tiles travel HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging) into a
// ring of kBufs buffers, kAhead = 3 tiles ahead.  A buffer has two regions: the first
// 1024 bytes of each of the 32 rows (dims 0..511) at a stride of 65 16-byte
// slots, one row per load instruction, and the last 128 bytes (dims 512..575)
// at a stride of 9 slots, four rows per load instruction.  Every source
// address is a wave-uniform row pointer plus a fixed lane offset.
//
// Within each 16-token half-tile, MFMA row m holds token perm16(m), which
// interleaves even and odd tokens so that, in a model of 32 four-byte LDS
// banks, the 8 rows read together by a ds_read_b128 of K fall on 8 different
// 16-byte bank groups (strides 65 and 9 are 1 mod 8) and the four rows read
// by each 16-lane ds_read_b64_tr_b16 group of V are 8 banks apart.  (Measured
// on gfx950, these strided reads still cost about 8 clocks per b128 and per
// tr16 instruction, against about 6 for a lane-contiguous b128.)  K operands
// are ds_read_b128 of 8 contiguous dims of one token; V^T operands come from
// ds_read_b64_tr_b16, whose 16-lane transpose turns four 16-column row
// segments into one column of 4 tokens per lane, which is exactly the V^T
// MFMA operand.
#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
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
constexpr int kAhead = kBufs - 1;           // tiles in flight ahead of the one computed
constexpr int kLoads = kRowsPerWave + kRowsPerWave / 4;  // load instructions per wave per tile
constexpr float kHeadroom = 64.0f;  // max log2 growth of P over the reference

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

// Token (within a 16-token half-tile) held by MFMA row m = 4a + i:
// a = 0 -> 0,2,4,6; a = 1 -> 1,3,5,7; a = 2 -> 8,..,14; a = 3 -> 9,..,15.
__device__ __forceinline__ int perm16(int m) { return ((m >> 2) & 1) + 2 * (m & 3) + 8 * (m >> 3); }

// PAGED: rows are found through the block table (paged cache layout).
template <bool PAGED>
__global__ __launch_bounds__(kThreads) void mla_mfma_kernel(PartialArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int lane = threadIdx.x & 63;
  // wave index as a scalar, so everything derived from it stays wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;

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

  // Q^T operands: [head block][18 chunks of 32 dims]; lane (n, g) holds head
  // 16*hb + n, dims 32c + 8g .. 32c + 8g + 7.
  bf16x8_t qop[2][18];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + (qrow0 + head0 + 16 * hb + r16) * kDqk;
#pragma unroll
    for (int c = 0; c < 18; ++c) {
      const uint4 v = *reinterpret_cast<const uint4*>(qrow + 32 * c + 8 * g);
      qop[hb][c] = as_bf16x8(v.x, v.y, v.z, v.w);
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
  const int tl_row = lane / 9;
  const int tl_chunk = (lane % 9) == 8 ? 7 : lane % 9;
  const uint32_t tl_off = (uint32_t)(kMainRowBytes + tl_chunk * 16);

  // Issue the direct-to-LDS loads of tile `tile` into buffer `buf`: this
  // wave's kRowsPerWave rows.  Rows past the shard end (last tile only) are
  // clamped to its last row.
  auto issue = [&](int tile, int buf) {
    const int64_t base = s0 + (int64_t)tile * kTile;
    const uint32_t bufaddr = lds0 + (uint32_t)(buf * kBufBytes);
    const int64_t g0 = base + kRowsPerWave * wave;   // this wave's first row (8-aligned)
    if (g0 + kRowsPerWave - 1 <= last) {
      // all 8 rows inside the shard; an aligned 8-row group is 8 consecutive
      // physical rows in every layout
      const uint8_t* src = kdata + hrow(g0) * kRowBytes;
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
                  kdata + hrow(row) * kRowBytes, (uint32_t)(lane * 16));
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
        int64_t row = row0 + tl_row;
        row = row < last ? row : last;
        const uint32_t off = (uint32_t)((row - rb) * kRowBytes) + tl_off;
        if (lane < 36) lds_dma16<true>(m0, kdata + hrow(rb) * kRowBytes, off);
      }
    }
  };

  // Per-lane LDS read offsets within a buffer.
  const int pk = perm16(r16);                  // token of this lane's K operand row
  const uint32_t k_main = (uint32_t)((pk * kMainStride + g) * 16);
  const uint32_t k_tail = (uint32_t)(kMainBytes + (pk * kTailStride + g) * 16);
  const int rr = r16 >> 2;                     // row of the lane's 4x16 transpose group
  const int q = r16 & 3;                       // 4-column piece of the 16 columns
  const uint32_t v_off =
      (uint32_t)((perm16(4 * g + rr) * kMainStride + (q >> 1)) * 16 + (q & 1) * 8);
  // token (within the tile) of each of the lane's 8 logits, for masking
  int tok[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) tok[e] = 16 * (e >> 2) + perm16(4 * g + (e & 3));

  f32x4_t acc[2][32];
  float m2[2], lsum[2];

  // Pass structure.  The accumulating pass fixes each head's reference max
  // at its first tile and never rescales the accumulator; weights may grow to
  // 2^kHeadroom before that is unsafe.  If any tile of the shard exceeds its
  // reference by more than kHeadroom (in log2 units) the workgroup reruns the
  // shard: a logits-only pass finds each head's exact max, then the
  // accumulating pass runs again with that max as the reference.
  bool max_only = false;
  m2[0] = m2[1] = -INFINITY;
  for (;;) {
    if (!max_only) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        lsum[hb] = 0.f;
#pragma unroll
        for (int blk = 0; blk < 32; ++blk) acc[hb][blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    int overflow = 0;
#pragma unroll
    for (int t = 0; t < kAhead; ++t)
      if (t < ntiles) issue(t, t);
    for (int tile = 0; tile < ntiles; ++tile) {
      const int buf = tile % kBufs;
      // this tile's loads are done once at most those of the tiles after it
      // remain in flight (s_waitcnt simm16 on gfx9: vmcnt in bits 3:0 and
      // 15:14, expcnt 6:4, lgkmcnt 11:8)
      const int after = ntiles - 1 - tile;
      if (after >= 2) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kLoads));
      } else if (after == 1) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoads));
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      }
      __builtin_amdgcn_s_barrier();
      // the buffer of tile + kAhead was last read in tile - 1, which every
      // wave has finished at the barrier above
      if (tile + kAhead < ntiles) issue(tile + kAhead, (tile + kAhead) % kBufs);
      const uint8_t* tb = smem + buf * kBufBytes;
      const int nvalid = (int)(s1 - (s0 + (int64_t)tile * kTile));   // > kTile except at the end

      // ---- logits for both 16-token halves and both head blocks; K operands
      // are read two chunks ahead of the MFMAs that use them
      f32x4_t s[2][2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) s[u][hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      auto kread = [&](int c, int u) {
        const uint8_t* p = c < 16 ? tb + k_main + (16 * u * kMainStride + 4 * c) * 16
                                  : tb + k_tail + (16 * u * kTailStride + 4 * (c - 16)) * 16;
        return *reinterpret_cast<const uint4*>(p);
      };
      uint4 ka0 = kread(0, 0), ka1 = kread(0, 1);
      uint4 kb0 = kread(1, 0), kb1 = kread(1, 1);
#pragma unroll
      for (int c = 0; c < 18; ++c) {
        const uint4 k0 = ka0, k1 = ka1;
        ka0 = kb0;
        ka1 = kb1;
        if (c + 2 < 18) {
          kb0 = kread(c + 2, 0);
          kb1 = kread(c + 2, 1);
        }
        const bf16x8_t a0 = as_bf16x8(k0.x, k0.y, k0.z, k0.w);
        const bf16x8_t a1 = as_bf16x8(k1.x, k1.y, k1.z, k1.w);
        s[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qop[0][c], s[0][0], 0, 0, 0);
        s[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qop[0][c], s[1][0], 0, 0, 0);
        s[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qop[1][c], s[0][1], 0, 0, 0);
        s[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qop[1][c], s[1][1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- softmax weights per head; lane (n, g) holds the logits of head n
      // for tokens tok[0..7]
      bf16x8_t pop[2], pol[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[4 * u + i] = s[u][hb][i];
        if (nvalid < kTile) {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = tok[e] < nvalid ? x[e] : -INFINITY;
        }
        float tmax = x[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, x[e]);
        const float tmax2 = rows4_max(tmax) * c2;
        if (max_only) {
          m2[hb] = fmaxf(m2[hb], tmax2);
          continue;
        }
        if (m2[hb] == -INFINITY) m2[hb] = tmax2;      // first tile: acc is still zero
        overflow |= (tmax2 > m2[hb] + kHeadroom);
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(fmaf(x[e], c2, -m2[hb]));  // masked logits give exp2(-inf) = 0
          lsum[hb] += p[e];
        }
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t b0 = __float_as_uint(p[2 * i]), b1 = __float_as_uint(p[2 * i + 1]);
          ph[i] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
          pl[i] = pack_bf16(p[2 * i] - __uint_as_float(b0 & 0xFFFF0000u),
                            p[2 * i + 1] - __uint_as_float(b1 & 0xFFFF0000u));
        }
        pop[hb] = as_bf16x8(ph[0], ph[1], ph[2], ph[3]);
        pol[hb] = as_bf16x8(pl[0], pl[1], pl[2], pl[3]);
      }
      if (max_only) continue;

      // ---- O^T += V^T P^T over 32 blocks of 16 value columns; V^T operands
      // are read two blocks ahead of their MFMAs
      const uint8_t* vl0 = tb + v_off;                        // tokens of half 0
      const uint8_t* vl1 = vl0 + 16 * kMainStride * 16;       // tokens of half 1
      auto vread = [&](const uint8_t* p, int blk) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 2 * blk * 16));
      };
      s16x4_t va0 = vread(vl0, 0), va1 = vread(vl1, 0);
      s16x4_t vb0 = vread(vl0, 1), vb1 = vread(vl1, 1);
#pragma unroll
      for (int blk = 0; blk < 32; ++blk) {
        const s16x4_t v0 = va0, v1 = va1;
        va0 = vb0;
        va1 = vb1;
        if (blk + 2 < 32) {
          vb0 = vread(vl0, blk + 2);
          vb1 = vread(vl1, blk + 2);
        }
        const uint2 w0 = __builtin_bit_cast(uint2, v0);
        const uint2 w1 = __builtin_bit_cast(uint2, v1);
        const bf16x8_t vop = as_bf16x8(w0.x, w0.y, w1.x, w1.y);
        acc[0][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[0], acc[0][blk], 0, 0, 0);
        acc[1][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[1], acc[1][blk], 0, 0, 0);
        acc[0][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pol[0], acc[0][blk], 0, 0, 0);
        acc[1][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pol[1], acc[1][blk], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // every wave is past its last LDS read before the buffers are refilled
    const int any_overflow = __syncthreads_or(overflow);
    if (max_only) {
      max_only = false;          // m2 now holds each head's exact max
      continue;
    }
    if (!any_overflow) break;
    max_only = true;
    m2[0] = m2[1] = -INFINITY;
  }

  // ---- write the normalized partial of this wave's 32 heads
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const float lt = rows4_sum(lsum[hb]);
    const bool empty = (m2[hb] == -INFINITY);
    const float inv = empty ? 0.0f : 1.0f / lt;
    const int h = head0 + 16 * hb + r16;
    float* orow = a.o_part + (orow0 + h) * kDv;
#pragma unroll
    for (int blk = 0; blk < 32; ++blk) {
      const f32x4_t v = acc[hb][blk] * inv;
      *reinterpret_cast<float4*>(orow + 16 * blk + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (g == 0)
      a.lse_part[orow0 + h] = empty ? -INFINITY : (m2[hb] + fast_log2(lt)) * kLn2;
  }
}

constexpr size_t kSmemBytes = (size_t)kBufs * kBufBytes;
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
