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
// Work split: one workgroup of 4 waves per (shard j, request b, KV head).  The
// shard is walked in 32-token tiles shared by all four waves; wave w owns heads
// 32w .. 32w+31, keeping their Q (144 VGPRs) and their O^T accumulator (32 heads
// x 512 dv, 256 AGPRs) in registers for the whole shard, so LDS traffic per
// cached token is 4 x (1152 + 1024) bytes, within the ~128 B/clk/CU LDS read
// rate at the HBM roof.
//
// Tiles travel HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging) into a
// ring of kBufs buffers, two tiles ahead.  Inside a buffer a tile row occupies
// 73 16-byte slots (1168 B: the 1152-byte row plus one pad slot), so 16 rows
// read at the same column start in 16 different bank groups, and every LDS
// read address is a per-lane base plus a compile-time offset.  Each
// wave-instruction of the loads fills 64 consecutive slots; lanes that land on
// a pad slot (or on the spare slots that round the tile up to 10 loads per
// thread) load a harmless in-shard chunk.  K operands are ds_read_b128 of 8
// contiguous dims of one token; V^T operands come from ds_read_b64_tr_b16,
// whose 16-lane transpose turns four 16-column row segments into one column of
// 4 tokens per lane, which is exactly the V^T MFMA operand.
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
constexpr int kHeads = 128;           // query heads per KV head
constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDqk * 2;   // 1152
constexpr int kChunks = kRowBytes / 16;  // 72 16-byte chunks per row
constexpr int kStride = kChunks + 1;     // 73 slots per row in LDS
constexpr int kTile = 32;
constexpr int kUsed = kTile * kStride;   // 2336 slots hold the tile
constexpr int kLoads = 10;               // direct-to-LDS loads per thread per tile
constexpr int kSlots = kLoads * kThreads;  // 2560 slots (40 KB) per buffer
constexpr int kBufs = 3;
constexpr float kHeadroom = 64.0f;  // max log2 growth of P over the reference

static_assert(kSlots >= kUsed, "buffer must hold the tile");

__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4_t v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  f32x2_t f = {x, y};
  bf16x2_t h = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, h);
}


__global__ __launch_bounds__(kThreads) void mla_mfma_kernel(PartialArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int lane = threadIdx.x & 63;
  // wave index as a scalar, so everything derived from it stays wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;

  int flat = blockIdx.x;
  const int kvh = flat % a.Hkv;
  flat /= a.Hkv;
  const int b = flat % a.B;
  const int j = flat / a.B;

  int64_t L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.S_max ? a.S_max : L);
  int64_t s0, s1;
  shard_range(L, a.kvp, j, &s0, &s1);
  const int ntiles = (int)((s1 - s0 + kTile - 1) / kTile);

  const int64_t slab = (int64_t)b * a.Hkv + kvh;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + slab * a.S_max * kRowBytes;
  const float c2 = a.scale_log2;
  const int head0 = kvh * kHeads + wave * 32;

  // Q^T operands: [head block][18 chunks of 32 dims]; lane (n, g) holds head
  // 16*hb + n, dims 32c + 8g .. 32c + 8g + 7.
  bf16x8_t qop[2][18];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.Hq + head0 + 16 * hb + r16) * kDqk;
#pragma unroll
    for (int c = 0; c < 18; ++c) {
      const uint4 v = *reinterpret_cast<const uint4*>(qrow + 32 * c + 8 * g);
      qop[hb][c] = as_bf16x8(v.x, v.y, v.z, v.w);
    }
  }
  // Q is in registers before any cache load is issued, so the only vector
  // memory operations in flight inside the tile loop are the tile loads whose
  // counts the loop waits on explicitly.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

  f32x4_t acc[2][32];
  float m2[2], lsum[2];
  const int64_t last = s1 - 1;

  // LDS byte address of the dynamic buffer ring.
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)smem;

  // Issue the direct-to-LDS loads of tile `tile` into buffer `buf` (with the
  // non-temporal hint: every cached byte is read once).  They are
  // written as inline asm so that the compiler does not treat every later LDS
  // read as possibly aliasing them (it would wait for all of them, including
  // the prefetch of the next tiles); the waits are explicit below.
  auto issue = [&](int tile, int buf) {
    const int64_t base = s0 + (int64_t)tile * kTile;
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      // the thread index goes through an opaque move so the ten per-lane
      // source offsets are recomputed per tile instead of being held live
      int tid;
      asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
      const int s = k * kThreads + tid;           // slot filled by this lane
      int t = s / kStride;
      int c = s - t * kStride;
      if (s >= kUsed) t = 0;                      // spare slot: any in-shard chunk
      if (c >= kChunks || s >= kUsed) c = 0;      // pad slot: likewise
      int64_t row = base + t;
      row = row < last ? row : last;
      const uint8_t* src = kbase + row * kRowBytes + c * 16;
      // M0 = LDS byte address of this wave's 64 consecutive slots
      const uint32_t dst = __builtin_amdgcn_readfirstlane(
          lds0 + (uint32_t)(buf * (kSlots * 16) + (k * kThreads + wave * 64) * 16));
      // (M0 is saved and restored around the load: the compiler owns it)
      uint32_t m0_saved;
      asm volatile(
          "s_mov_b32 %0, m0\n\t"
          "s_mov_b32 m0, %1\n\t"
          "s_nop 0\n\t"
          "global_load_lds_dwordx4 %2, off nt\n\t"
          "s_mov_b32 m0, %0"
          : "=&s"(m0_saved)
          : "s"(dst), "v"(src)
          : "memory");
    }
  };

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
    if (ntiles > 0) {
      issue(0, 0);
      if (ntiles > 1) issue(1, 1);
    }
    for (int tile = 0; tile < ntiles; ++tile) {
      const int buf = tile % kBufs;
      // this tile's loads are done once at most the next tile's remain
      // (s_waitcnt simm16 on gfx9: vmcnt in bits 3:0, expcnt 6:4, lgkmcnt 11:8)
      if (tile + 1 < ntiles) {
        __builtin_amdgcn_s_waitcnt(0x0F70 | kLoads);   // vmcnt(kLoads)
      } else {
        __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0)
      }
      __builtin_amdgcn_s_barrier();
      if (tile + 2 < ntiles) issue(tile + 2, (tile + 2) % kBufs);
      const uint8_t* tb = smem + buf * (kSlots * 16);
      const int64_t base = s0 + (int64_t)tile * kTile;

      // ---- logits for both 16-token halves and both head blocks, with the K
      // operands of chunk c+1 read while chunk c's MFMAs run
      f32x4_t s[2][2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) s[u][hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint8_t* kl = tb + (r16 * kStride + g) * 16;      // this lane's K base
      uint4 kn0 = *reinterpret_cast<const uint4*>(kl);
      uint4 kn1 = *reinterpret_cast<const uint4*>(kl + 16 * kStride * 16);
#pragma unroll
      for (int c = 0; c < 18; ++c) {
        const uint4 k0 = kn0, k1 = kn1;
        if (c + 1 < 18) {
          kn0 = *reinterpret_cast<const uint4*>(kl + 4 * (c + 1) * 16);
          kn1 = *reinterpret_cast<const uint4*>(kl + (16 * kStride + 4 * (c + 1)) * 16);
        }
        const bf16x8_t a0 = as_bf16x8(k0.x, k0.y, k0.z, k0.w);
        const bf16x8_t a1 = as_bf16x8(k1.x, k1.y, k1.z, k1.w);
        s[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qop[0][c], s[0][0], 0, 0, 0);
        s[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qop[0][c], s[1][0], 0, 0, 0);
        s[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qop[1][c], s[0][1], 0, 0, 0);
        s[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qop[1][c], s[1][1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- softmax weights per head (lane (n, g): tokens 16u + 4g + i)
      bf16x8_t pop[2], pol[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t t = base + 16 * u + 4 * g + i;
            x[4 * u + i] = (t < s1) ? s[u][hb][i] : -INFINITY;
          }
        float tmax = x[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, x[e]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float tmax2 = tmax * c2;
        if (max_only) {
          m2[hb] = fmaxf(m2[hb], tmax2);
          continue;
        }
        if (m2[hb] == -INFINITY) m2[hb] = tmax2;      // first tile: acc is still zero
        overflow |= (tmax2 > m2[hb] + kHeadroom);
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = fast_exp2(fmaf(x[e], c2, -m2[hb]));
          p[e] = (x[e] == -INFINITY) ? 0.0f : pe;
          lsum[hb] += p[e];
        }
        uint32_t ph[4], pl[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const uint32_t b0 = __float_as_uint(p[2 * rr]), b1 = __float_as_uint(p[2 * rr + 1]);
          ph[rr] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
          pl[rr] = pack_bf16(p[2 * rr] - __uint_as_float(b0 & 0xFFFF0000u),
                             p[2 * rr + 1] - __uint_as_float(b1 & 0xFFFF0000u));
        }
        pop[hb] = as_bf16x8(ph[0], ph[1], ph[2], ph[3]);
        pol[hb] = as_bf16x8(pl[0], pl[1], pl[2], pl[3]);
      }
      if (max_only) continue;

      // ---- O^T += V^T P^T over 32 blocks of 16 value columns, one block ahead
      const int rr = r16 >> 2;      // row of the 4x16 transpose group
      const int q = r16 & 3;        // 4-column piece within the 16 columns
      const uint8_t* vl0 = tb + ((4 * g + rr) * kStride + (q >> 1)) * 16 + (q & 1) * 8;
      const uint8_t* vl1 = vl0 + 16 * kStride * 16;
      s16x4_t vn0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)vl0);
      s16x4_t vn1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)vl1);
#pragma unroll
      for (int blk = 0; blk < 32; ++blk) {
        const s16x4_t v0 = vn0, v1 = vn1;
        if (blk + 1 < 32) {
          vn0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vl0 + 2 * (blk + 1) * 16));
          vn1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vl1 + 2 * (blk + 1) * 16));
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
    float lt = lsum[hb];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const bool empty = (m2[hb] == -INFINITY);
    const float inv = empty ? 0.0f : 1.0f / lt;
    const int h = head0 + 16 * hb + r16;
    float* orow = a.o_part + (((int64_t)j * a.B + b) * a.Hq + h) * kDv;
#pragma unroll
    for (int blk = 0; blk < 32; ++blk) {
      const f32x4_t v = acc[hb][blk] * inv;
      *reinterpret_cast<float4*>(orow + 16 * blk + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (g == 0)
      a.lse_part[((int64_t)j * a.B + b) * a.Hq + h] = empty ? -INFINITY : (m2[hb] + fast_log2(lt)) * kLn2;
  }
}

constexpr size_t kSmemBytes = (size_t)kBufs * kSlots * 16;

}  // namespace

bool mla_mfma_supports(const PartialArgs& a) {
  return a.q_bf16 && a.kv_format == kBF16 && a.v_aliases_k && a.Dqk == kDqk && a.Dv == kDv &&
         a.Hq / a.Hkv == kHeads;
}

hipError_t launch_partial_mla_mfma(const PartialArgs& a, hipStream_t stream) {
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(mla_mfma_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmemBytes);
    if (e != hipSuccess) return e;
    configured = true;
  }
  const int64_t blocks = (int64_t)a.kvp * a.B * a.Hkv;
  hipLaunchKernelGGL(mla_mfma_kernel, dim3((unsigned)blocks), dim3(kThreads), kSmemBytes, stream, a);
  return hipGetLastError();
}

}  // namespace kvd
