// Split-KV partial attention on the vector ALUs: the general path.
//
// Handles every KV format for head widths 64, 128 and 256 (MXFP4: 128, 256)
// and any query-head group size G.  One workgroup (4 waves) owns one
// (shard j, request b, KV head, chunk of up to HC query heads, query token).  Each wave is
// four DPP rows of 16 lanes; a row owns one cached token at a time and each
// lane holds D/16 consecutive elements of that token's K and V rows, so a row
// streams whole cache rows with coalesced 4-64 byte loads.  The 16 rows of the
// workgroup take tokens s0 + r, s0 + r + 16, ... of the shard.
//
// Per token a row forms the logit of every query head of its chunk (a dot
// product over its D/16 elements, summed across the row with DPP), then
// updates its running softmax state (m, l, acc) in the log2 domain.  After the
// shard is consumed the 16 row states are combined (wave shuffles, then LDS)
// with the same max/sum algebra, and the normalized partial o and its
// natural-log lse are written.
#include "kvd_device.hpp"
#include "kvd_internal.hpp"

namespace kvd {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = kThreads / 16;

// HC: query heads per workgroup.  DEPTH: tokens per row whose loads are in
// flight together (2 for full grids; 8 for small ones, where every row has
// many tokens to walk and load latency, not throughput, sets the time).
template <int KV, int DQK, int DV, int HC, bool QBF16, bool ALIAS, int DEPTH>
__global__ __launch_bounds__(kThreads) void partial_valu_kernel(PartialArgs a) {
  constexpr int EK = DQK / 16;
  constexpr int EV = DV / 16;
  constexpr int BITS = KvTraits<KV>::kBitsPerElem;
  constexpr int KLANE = EK * BITS / 8;  // bytes per lane per token
  constexpr int VLANE = EV * BITS / 8;
  constexpr int64_t KROW = (int64_t)DQK * BITS / 8;  // bytes per cached token
  constexpr int64_t VROW = ALIAS ? KROW : (int64_t)DV * BITS / 8;
  constexpr int KW = KLANE / 4;
  constexpr int VW = VLANE / 4;

  __shared__ float sh_acc[4][HC][DV];
  __shared__ float sh_m[4][HC];
  __shared__ float sh_l[4][HC];

  const int G = a.Hq / a.Hkv;
  const int nhc = (G + HC - 1) / HC;
  // unit (shard j, request b, KV head kvh, head chunk hc) and query token qt
  int64_t unit;
  int qt;
  if (!unit_token(blockIdx.x, (int64_t)a.kvp * a.B * a.Hkv * nhc, a.T, &unit, &qt)) return;
  const int hc = (int)(unit % nhc);
  int64_t flat = unit / nhc;
  const int kvh = (int)(flat % a.Hkv);
  flat /= a.Hkv;
  const int b = (int)(flat % a.B);
  const int j = (int)(flat / a.B);
  const int h0 = kvh * G + hc * HC;
  const int64_t qrow0 = ((int64_t)b * a.T + qt) * a.Hq;                // q row of head h: qrow0 + h
  const int64_t orow0 = (((int64_t)j * a.B + b) * a.T + qt) * a.Hq;    // o_part / lse_part row
  const int nh = min(HC, G - hc * HC);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 15;
  const int row = wave * 4 + (lane >> 4);

  const ShardSpan span = shard_span(a.layout, a.seq_lens[b], a.T, qt, a.S_max, a.kvp, a.B, a.Hkv, j, b, kvh);
  const int64_t s0 = span.s0, s1 = span.s1;
  const int64_t slab = span.slab;                  // cache block of this shard
  const int64_t bh = (int64_t)b * a.Hkv + kvh;     // fp8 scales are per (request, KV head)

  // cache arrays viewed as rows; token t of this shard is physical row
  // phys_row(t) (slab * S_max + t, or through the block table when paged)
  const uint8_t* kp = static_cast<const uint8_t*>(a.k) + li * KLANE;
  const uint8_t* vp = ALIAS ? static_cast<const uint8_t*>(a.k) + li * VLANE
                            : static_cast<const uint8_t*>(a.v) + li * VLANE;
  const uint8_t* ksp = nullptr;
  const uint8_t* vsp = nullptr;
  float kscale = 1.0f, vscale = 1.0f;
  if constexpr (KV == kFP8) {
    kscale = static_cast<const float*>(a.k_scale)[bh];
    vscale = ALIAS ? kscale : static_cast<const float*>(a.v_scale)[bh];
  }
  if constexpr (KV == kMXFP4) {
    ksp = static_cast<const uint8_t*>(a.k_scale) + (li * EK) / 32;
    vsp = ALIAS ? static_cast<const uint8_t*>(a.k_scale) + (li * EV) / 32
                : static_cast<const uint8_t*>(a.v_scale) + (li * EV) / 32;
  }
  constexpr int64_t KSROW = DQK / 32;
  constexpr int64_t VSROW = ALIAS ? DQK / 32 : DV / 32;

  // Query slice of every head of the chunk, pre-multiplied into the log2 domain.
  float qs[HC][EK];
  {
    const float qmul = a.scale_log2 * kscale;
#pragma unroll
    for (int i = 0; i < HC; ++i) {
      const int h = h0 + (i < nh ? i : nh - 1);
      const int64_t off = (qrow0 + h) * DQK + li * EK;
      if constexpr (QBF16) {
        uint32_t w[EK / 2];
#pragma unroll
        for (int e = 0; e < EK / 2; ++e)
          w[e] = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.q) + off)[e];
#pragma unroll
        for (int e = 0; e < EK / 2; ++e) {
          qs[i][2 * e] = bf16_lo(w[e]) * qmul;
          qs[i][2 * e + 1] = bf16_hi(w[e]) * qmul;
        }
      } else {
#pragma unroll
        for (int e = 0; e < EK; ++e) qs[i][e] = static_cast<const float*>(a.q)[off + e] * qmul;
      }
    }
  }

  float m[HC], l[HC], acc[HC][EV];
#pragma unroll
  for (int i = 0; i < HC; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.0f;
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[i][e] = 0.0f;
  }

  auto process = [&](const uint32_t* kw, const uint32_t* vw, float ks, float vs) {
    float kf[EK], vf[EV];
    decode_elems<KV, EK>(kw, ks, kf);
    decode_elems<KV, EV>(vw, vs, vf);
#pragma unroll
    for (int i = 0; i < HC; ++i) {
      float d = 0.0f;
#pragma unroll
      for (int e = 0; e < EK; ++e) d = fmaf(qs[i][e], kf[e], d);
      d = row16_sum(d);
      const float mn = fmaxf(m[i], d);
      const float al = fast_exp2(m[i] - mn);
      const float p = fast_exp2(d - mn);
      l[i] = fmaf(l[i], al, p);
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[i][e] = fmaf(acc[i][e], al, p * vf[e]);
      m[i] = mn;
    }
  };

  auto load = [&](int64_t tok, uint32_t* kw, uint32_t* vw, float* ks, float* vs) {
    const int64_t t = phys_row(a, b, kvh, slab, tok);
    load_dwords<KLANE>(kp + t * KROW, kw);
    load_dwords<VLANE>(vp + t * VROW, vw);
    if constexpr (KV == kMXFP4) {
      *ks = e8m0_to_f32(stream_load1(ksp + t * KSROW));
      *vs = e8m0_to_f32(stream_load1(vsp + t * VSROW));
    } else {
      *ks = 1.0f;
      *vs = 1.0f;
    }
  };

  int64_t t = s0 + row;
  for (; t + (DEPTH - 1) * kRows < s1; t += DEPTH * kRows) {
    uint32_t kw[DEPTH][KW], vw[DEPTH][VW];
    float ks[DEPTH], vs[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) load(t + d * kRows, kw[d], vw[d], &ks[d], &vs[d]);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) process(kw[d], vw[d], ks[d], vs[d]);
  }
  for (; t < s1; t += kRows) {
    uint32_t kw0[KW], vw0[VW];
    float ks0, vs0;
    load(t, kw0, vw0, &ks0, &vs0);
    process(kw0, vw0, ks0, vs0);
  }

  // Combine the four rows of this wave (lanes l, l^16, l^32, l^48 hold the
  // same element slice).
#pragma unroll
  for (int i = 0; i < HC; ++i) {
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float mo = __shfl_xor(m[i], off);
      const float lo = __shfl_xor(l[i], off);
      const float M = fmaxf(m[i], mo);
      const float f1 = rescale_weight(m[i], M);
      const float f2 = rescale_weight(mo, M);
      l[i] = l[i] * f1 + lo * f2;
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[i][e] = acc[i][e] * f1 + __shfl_xor(acc[i][e], off) * f2;
      m[i] = M;
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int i = 0; i < HC; ++i) {
#pragma unroll
      for (int e = 0; e < EV; ++e) sh_acc[wave][i][li * EV + e] = acc[i][e];
      if (li == 0) {
        sh_m[wave][i] = m[i];
        sh_l[wave][i] = l[i];
      }
    }
  }
  __syncthreads();

  // Combine the four waves and write the normalized partial.
  for (int idx = tid; idx < nh * DV; idx += kThreads) {
    const int i = idx / DV;
    const int d = idx - i * DV;
    float M = sh_m[0][i];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sh_m[w][i]);
    float o = 0.0f;
    if (M != -INFINITY) {
      float lsum = 0.0f, osum = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = rescale_weight(sh_m[w][i], M);
        lsum += sh_l[w][i] * f;
        osum += sh_acc[w][i][d] * f;
      }
      o = osum / lsum * vscale;
    }
    a.o_part[(orow0 + h0 + i) * DV + d] = o;
  }
  for (int i = tid; i < nh; i += kThreads) {
    float M = sh_m[0][i];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sh_m[w][i]);
    float lse = -INFINITY;
    if (M != -INFINITY) {
      float lsum = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) lsum += sh_l[w][i] * rescale_weight(sh_m[w][i], M);
      lse = (M + fast_log2(lsum)) * kLn2;
    }
    a.lse_part[orow0 + h0 + i] = lse;
  }
}

template <int D>
constexpr int head_chunk() {
  return D <= 128 ? 8 : 4;
}

// A grid of fewer workgroups than the chip has compute units (a few shards of
// a few requests) runs one query head per workgroup with eight tokens in
// flight per row: more workgroups, each with a short latency-bound walk.
constexpr int64_t kSmallGrid = 256;

int64_t grid_units(const PartialArgs& a, int hc) {
  const int G = a.Hq / a.Hkv;
  return (int64_t)a.kvp * a.B * a.Hkv * ((G + hc - 1) / hc) * a.T;
}

bool small_grid(const PartialArgs& a) { return grid_units(a, a.Dqk <= 128 ? 8 : 4) < kSmallGrid; }

using KernelFn = void (*)(PartialArgs);

template <int KV, int D, bool QBF16, bool ALIAS>
KernelFn pick3(bool small) {
  if (small) return partial_valu_kernel<KV, D, D, 1, QBF16, ALIAS, 8>;
  return partial_valu_kernel<KV, D, D, head_chunk<D>(), QBF16, ALIAS, 2>;
}

template <int KV, int D>
KernelFn pick2(bool qbf16, bool alias, bool small) {
  if (qbf16) return alias ? pick3<KV, D, true, true>(small) : pick3<KV, D, true, false>(small);
  return alias ? pick3<KV, D, false, true>(small) : pick3<KV, D, false, false>(small);
}

template <int KV>
KernelFn pick1(int D, bool qbf16, bool alias, bool small) {
  if constexpr (KV != kMXFP4) {
    if (D == 64) return pick2<KV, 64>(qbf16, alias, small);
  }
  if (D == 128) return pick2<KV, 128>(qbf16, alias, small);
  if (D == 256) return pick2<KV, 256>(qbf16, alias, small);
  return nullptr;
}

KernelFn pick(const PartialArgs& a) {
  const bool qb = a.q_bf16 != 0, al = a.v_aliases_k != 0, sm = small_grid(a);
  switch (a.kv_format) {
    case kF32: return pick1<kF32>(a.Dqk, qb, al, sm);
    case kBF16: return pick1<kBF16>(a.Dqk, qb, al, sm);
    case kFP8: return pick1<kFP8>(a.Dqk, qb, al, sm);
    case kMXFP4: return pick1<kMXFP4>(a.Dqk, qb, al, sm);
    default: return nullptr;
  }
}

}  // namespace

bool valu_supports(const PartialArgs& a) {
  if (a.Dqk != a.Dv) return false;
  return pick(a) != nullptr;
}

hipError_t launch_partial_valu(const PartialArgs& a, hipStream_t stream) {
  KernelFn fn = pick(a);
  if (fn == nullptr) return hipErrorInvalidValue;
  const int G = a.Hq / a.Hkv;
  const int hc = small_grid(a) ? 1 : (a.Dqk <= 128 ? 8 : 4);
  const int64_t blocks = unit_token_blocks((int64_t)a.kvp * a.B * a.Hkv * ((G + hc - 1) / hc), a.T);
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvd
