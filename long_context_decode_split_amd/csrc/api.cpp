// C ABI of libkvd.so (declared in include/kvd.h): host-side validation,
// kernel selection and launches.  No device memory is read or written here and
// nothing is allocated at run time; every launch goes onto the caller's
// stream.  The one piece of device memory the library owns is the static
// partials array of kvd_decode_noalloc (below), which the code-object loader
// places on each device the library runs on.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "kvd.h"
#include "kvd_internal.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return KVD_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kMaxKvp = 4096;
constexpr int kMaxQTokens = 65536;
constexpr size_t kWorkspaceAlign = 256;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Bits per cached element of each format.
int elem_bits(int kv) {
  switch (kv) {
    case KVD_F32: return 32;
    case KVD_BF16: return 16;
    case KVD_FP8_E4M3: return 8;
    case KVD_MXFP4: return 4;
    default: return 0;
  }
}

// Query (and new) tokens per request: q_tokens, with 0 meaning 1.
int64_t tokens(const kvd_problem* p) { return p->q_tokens == 0 ? 1 : p->q_tokens; }

// Shape and format checks shared by every entry point taking a kvd_problem.
int check_problem(const kvd_problem* p) {
  if (p == nullptr) return fail(KVD_ERR_INVALID, "problem is NULL");
  if (p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->Dqk < 1 || p->Dv < 1)
    return fail(KVD_ERR_INVALID, "B, Hq, Hkv, Dqk, Dv must be >= 1 (got %d, %d, %d, %d, %d)", p->B,
                p->Hq, p->Hkv, p->Dqk, p->Dv);
  if (p->Hq % p->Hkv != 0)
    return fail(KVD_ERR_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
  if (p->S_max < 1) return fail(KVD_ERR_INVALID, "S_max must be >= 1");
  if (p->kvp < 1 || p->kvp > kMaxKvp)
    return fail(KVD_ERR_INVALID, "kvp must be in [1, %d] (got %d)", kMaxKvp, p->kvp);
  if (p->q_dtype != KVD_F32 && p->q_dtype != KVD_BF16)
    return fail(KVD_ERR_INVALID, "q_dtype must be KVD_F32 or KVD_BF16");
  if (p->q_tokens < 0 || p->q_tokens > kMaxQTokens)
    return fail(KVD_ERR_INVALID, "q_tokens must be in [0, %d] (got %d)", kMaxQTokens, p->q_tokens);
  if (elem_bits(p->kv_dtype) == 0) return fail(KVD_ERR_INVALID, "unknown kv_dtype %d", p->kv_dtype);
  if (!(p->sm_scale >= 0.0f) || !std::isfinite(p->sm_scale))
    return fail(KVD_ERR_INVALID, "sm_scale must be finite and >= 0");
  if (p->kv_dtype == KVD_MXFP4 && (p->Dqk % 32 != 0 || p->Dv % 32 != 0))
    return fail(KVD_ERR_INVALID, "MXFP4 needs Dqk and Dv multiples of 32");
  if (p->v_aliases_k && p->Dv > p->Dqk)
    return fail(KVD_ERR_INVALID, "v_aliases_k needs Dv <= Dqk");
  if (p->layout != KVD_LAYOUT_CONTIGUOUS && p->layout != KVD_LAYOUT_STRIPED &&
      p->layout != KVD_LAYOUT_STAGGERED16 && p->layout != KVD_LAYOUT_PAGED)
    return fail(KVD_ERR_INVALID, "unknown layout %d", p->layout);
  double rows;   // cache rows per KV head and request slot, for the size check
  if (p->layout == KVD_LAYOUT_PAGED) {
    const int bl = p->block_len;
    if (bl < 16 || bl > (1 << 20) || (bl & (bl - 1)) != 0)
      return fail(KVD_ERR_INVALID, "block_len must be a power of two in [16, 2^20] (got %d)", bl);
    if (p->max_blocks < 1) return fail(KVD_ERR_INVALID, "max_blocks must be >= 1");
    if (p->num_blocks < 1) return fail(KVD_ERR_INVALID, "num_blocks must be >= 1");
    if (p->block_table == nullptr || !aligned(p->block_table, 4))
      return fail(KVD_ERR_INVALID, "block_table must be non-NULL and 4-byte aligned");
    if ((double)p->max_blocks * bl > 2.0e9) return fail(KVD_ERR_UNSUPPORTED, "max_blocks*block_len too large");
    rows = (double)p->num_blocks * bl / p->B;
  } else {
    rows = (p->layout == KVD_LAYOUT_CONTIGUOUS ? 1.0 : (double)p->kvp) * (double)p->S_max;
  }
  // every byte offset into the cache must fit in int64
  const double cache_bytes = (double)p->B * p->Hkv * rows *
                             (double)(p->Dqk > p->Dv ? p->Dqk : p->Dv) * elem_bits(p->kv_dtype) / 8;
  if (cache_bytes > 9.0e18) return fail(KVD_ERR_INVALID, "cache too large to index");
  const double part_elems = (double)p->kvp * p->B * tokens(p) * p->Hq * (double)p->Dv;
  if (part_elems > 2.0e9) return fail(KVD_ERR_UNSUPPORTED, "kvp*B*q_tokens*Hq*Dv too large");
  // workgroup ids (at most one per shard, request, query token and query
  // head, plus 8 units of padding per token) and append ids fit in int32
  if (((double)p->kvp * p->B * p->Hq + 8.0) * tokens(p) > 2.0e9 ||
      (double)p->B * tokens(p) * p->Hkv * 2.0 > 2.0e9)
    return fail(KVD_ERR_UNSUPPORTED, "kvp*B*Hq*q_tokens too large");
  return KVD_OK;
}

int check_tensors(const kvd_problem* p, const void* q, kvd_kv k, kvd_kv v, const int32_t* seq_lens,
                  bool need_q16 = true) {
  if (q == nullptr || k.data == nullptr || seq_lens == nullptr)
    return fail(KVD_ERR_INVALID, "q, k.data and seq_lens must be non-NULL");
  if ((need_q16 && !aligned(q, 16)) || !aligned(k.data, 16))
    return fail(KVD_ERR_INVALID, "q and k.data must be 16-byte aligned");
  if (!aligned(seq_lens, 4)) return fail(KVD_ERR_INVALID, "seq_lens must be 4-byte aligned");
  const bool scaled = p->kv_dtype == KVD_FP8_E4M3 || p->kv_dtype == KVD_MXFP4;
  if (scaled && k.scale == nullptr) return fail(KVD_ERR_INVALID, "k.scale is required for fp8/MXFP4");
  if (!scaled && k.scale != nullptr) return fail(KVD_ERR_INVALID, "k.scale must be NULL for f32/bf16");
  if (scaled && !aligned(k.scale, 4)) return fail(KVD_ERR_INVALID, "k.scale must be 4-byte aligned");
  if (p->v_aliases_k) {
    if (v.data != nullptr || v.scale != nullptr)
      return fail(KVD_ERR_INVALID, "v must be {NULL, NULL} when v_aliases_k is set");
  } else {
    if (v.data == nullptr) return fail(KVD_ERR_INVALID, "v.data must be non-NULL");
    if (!aligned(v.data, 16)) return fail(KVD_ERR_INVALID, "v.data must be 16-byte aligned");
    if (scaled && v.scale == nullptr) return fail(KVD_ERR_INVALID, "v.scale is required for fp8/MXFP4");
    if (!scaled && v.scale != nullptr) return fail(KVD_ERR_INVALID, "v.scale must be NULL for f32/bf16");
    if (scaled && !aligned(v.scale, 4)) return fail(KVD_ERR_INVALID, "v.scale must be 4-byte aligned");
  }
  return KVD_OK;
}

// Paged caches: the block table and log2(block_len); S_max becomes the
// request capacity max_blocks * block_len, which bounds every length.
template <class Args>
void set_paging(const kvd_problem* p, Args* a) {
  a->block_table = nullptr;
  a->log2_block = 0;
  a->max_blocks = 0;
  a->num_blocks = 0;
  if (p->layout != KVD_LAYOUT_PAGED) return;
  int lg = 0;
  while ((1 << lg) < p->block_len) ++lg;
  a->block_table = p->block_table;
  a->log2_block = lg;
  a->max_blocks = p->max_blocks;
  a->num_blocks = p->num_blocks;
  a->S_max = (int64_t)p->max_blocks << lg;
}

kvd::PartialArgs make_args(const kvd_problem* p, const void* q, kvd_kv k, kvd_kv v,
                           const int32_t* seq_lens, float* o_part, float* lse_part) {
  kvd::PartialArgs a{};
  a.q = q;
  a.k = k.data;
  a.k_scale = k.scale;
  a.v = p->v_aliases_k ? k.data : v.data;
  a.v_scale = p->v_aliases_k ? k.scale : v.scale;
  a.seq_lens = seq_lens;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.B = p->B;
  a.Hq = p->Hq;
  a.Hkv = p->Hkv;
  a.Dqk = p->Dqk;
  a.Dv = p->Dv;
  a.kvp = p->kvp;
  a.T = (int32_t)tokens(p);
  a.S_max = p->S_max;
  set_paging(p, &a);
  a.q_bf16 = p->q_dtype == KVD_BF16;
  a.kv_format = p->kv_dtype;
  a.v_aliases_k = p->v_aliases_k != 0;
  const double s = p->sm_scale > 0.0f ? (double)p->sm_scale : 1.0 / std::sqrt((double)p->Dqk);
  a.scale_log2 = (float)(s * 1.4426950408889634);
  a.layout = p->layout;
  return a;
}

enum class Path { kNone, kValu, kGqaMfma, kMlaMfma };

// KVD_PATH=valu restricts kernel selection to the general vector-ALU path
// (for cross-checking the matrix-core kernels); anything else selects the
// fastest kernel that handles the problem.
bool valu_only() {
  static const bool v = [] {
    const char* e = std::getenv("KVD_PATH");
    return e != nullptr && std::strcmp(e, "valu") == 0;
  }();
  return v;
}

Path choose(const kvd::PartialArgs& a) {
  if (!valu_only()) {
    if (kvd::mla_mfma_supports(a)) return Path::kMlaMfma;
    if (kvd::gqa_mfma_supports(a)) return Path::kGqaMfma;
  }
  if (kvd::valu_supports(a)) return Path::kValu;
  return Path::kNone;
}

int launch_partial(const kvd_problem* p, const void* q, kvd_kv k, kvd_kv v, const int32_t* seq_lens,
                   float* o_part, float* lse_part, hipStream_t stream) {
  const kvd::PartialArgs a = make_args(p, q, k, v, seq_lens, o_part, lse_part);
  hipError_t e;
  switch (choose(a)) {
    case Path::kMlaMfma: e = kvd::launch_partial_mla_mfma(a, stream); break;
    case Path::kGqaMfma: e = kvd::launch_partial_gqa_mfma(a, stream); break;
    case Path::kValu: e = kvd::launch_partial_valu(a, stream); break;
    default:
      return fail(KVD_ERR_UNSUPPORTED,
                  "no kernel for Hq=%d Hkv=%d Dqk=%d Dv=%d kv_dtype=%d q_dtype=%d v_aliases_k=%d",
                  p->Hq, p->Hkv, p->Dqk, p->Dv, p->kv_dtype, p->q_dtype, p->v_aliases_k);
  }
  if (e != hipSuccess) return fail(KVD_ERR_HIP, "partial launch failed: %s", hipGetErrorString(e));
  return ok();
}

int check_merge(int32_t kvp, int64_t rows, int32_t Dv, const float* o_part, const float* lse_part,
                float* o, float* lse) {
  if (kvp < 1 || kvp > kMaxKvp) return fail(KVD_ERR_INVALID, "kvp must be in [1, %d]", kMaxKvp);
  if (rows < 0) return fail(KVD_ERR_INVALID, "rows must be >= 0");
  if (Dv < 4 || Dv % 4 != 0) return fail(KVD_ERR_INVALID, "Dv must be a positive multiple of 4");
  if ((double)rows * (Dv / 4) > 2.0e9) return fail(KVD_ERR_UNSUPPORTED, "rows*Dv too large");
  if (rows == 0) return KVD_OK;
  if (o_part == nullptr || lse_part == nullptr || o == nullptr || lse == nullptr)
    return fail(KVD_ERR_INVALID, "o_part, lse_part, o and lse must be non-NULL");
  if (!aligned(o_part, 16) || !aligned(o, 16))
    return fail(KVD_ERR_INVALID, "o_part and o must be 16-byte aligned");
  if (!aligned(lse_part, 4) || !aligned(lse, 4))
    return fail(KVD_ERR_INVALID, "lse_part and lse must be 4-byte aligned");
  return KVD_OK;
}

size_t workspace_o_bytes(const kvd_problem* p) {
  return round_up((size_t)p->kvp * p->B * tokens(p) * p->Hq * p->Dv * sizeof(float), kWorkspaceAlign);
}

size_t workspace_lse_bytes(const kvd_problem* p) {
  return round_up((size_t)p->kvp * p->B * tokens(p) * p->Hq * sizeof(float), kWorkspaceAlign);
}

}  // namespace

// Shard partials of kvd_decode_noalloc: one copy per device (the loader
// allocates it with the code object; it lives until the process ends).  In
// host code this name is only a handle for hipGetSymbolAddress: kernels and
// copies take the device address that call returns (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[KVD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr with an error message
// if the lookup fails.
void* noalloc_scratch(int* status) {
  static std::once_flag once[kMaxDevices];
  static void* addr[kMaxDevices];
  static hipError_t err[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *status = fail(KVD_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = fail(KVD_ERR_UNSUPPORTED, "device %d is beyond the %d devices kvd_decode_noalloc serves", dev,
                   kMaxDevices);
    return nullptr;
  }
  std::call_once(once[dev], [dev] {
    void* p = nullptr;
    err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    addr[dev] = err[dev] == hipSuccess ? p : nullptr;
  });
  if (err[dev] != hipSuccess || addr[dev] == nullptr) {
    *status = fail(KVD_ERR_HIP, "hipGetSymbolAddress of the static partials failed on device %d: %s", dev,
                   hipGetErrorString(err[dev]));
    return nullptr;
  }
  return addr[dev];
}

}  // namespace

extern "C" {

int kvd_abi_version(void) { return KVD_ABI_VERSION; }

const char* kvd_status_string(int status) {
  switch (status) {
    case KVD_OK: return "KVD_OK";
    case KVD_ERR_INVALID: return "KVD_ERR_INVALID: malformed argument";
    case KVD_ERR_UNSUPPORTED: return "KVD_ERR_UNSUPPORTED: no kernel for this problem";
    case KVD_ERR_HIP: return "KVD_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown kvd status";
  }
}

const char* kvd_last_error(void) { return g_last_error; }

int kvd_decode_partial(const kvd_problem* p, const void* q, kvd_kv k, kvd_kv v,
                       const int32_t* seq_lens, float* o_part, float* lse_part,
                       kvd_stream_t stream) {
  int s = check_problem(p);
  if (s != KVD_OK) return s;
  s = check_tensors(p, q, k, v, seq_lens);
  if (s != KVD_OK) return s;
  if (o_part == nullptr || lse_part == nullptr)
    return fail(KVD_ERR_INVALID, "o_part and lse_part must be non-NULL");
  if (!aligned(o_part, 16) || !aligned(lse_part, 4))
    return fail(KVD_ERR_INVALID, "o_part must be 16-byte and lse_part 4-byte aligned");
  return launch_partial(p, q, k, v, seq_lens, o_part, lse_part, reinterpret_cast<hipStream_t>(stream));
}

int kvd_lse_merge(int32_t kvp, int64_t rows, int32_t Dv, const float* o_part, const float* lse_part,
                  float* o, float* lse, kvd_stream_t stream) {
  int s = check_merge(kvp, rows, Dv, o_part, lse_part, o, lse);
  if (s != KVD_OK) return s;
  hipError_t e = kvd::launch_lse_merge(kvp, rows, Dv, o_part, lse_part, o, lse,
                                       reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVD_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

int kvd_append_kv(const kvd_problem* p, const float* k_new, const float* v_new,
                  const int32_t* positions, kvd_kv k, kvd_kv v, kvd_stream_t stream) {
  int s = check_problem(p);
  if (s != KVD_OK) return s;
  if (k_new == nullptr || positions == nullptr)
    return fail(KVD_ERR_INVALID, "k_new and positions must be non-NULL");
  if (!aligned(k_new, 4) || !aligned(positions, 4))
    return fail(KVD_ERR_INVALID, "k_new and positions must be 4-byte aligned");
  if (p->v_aliases_k) {
    if (v_new != nullptr) return fail(KVD_ERR_INVALID, "v_new must be NULL when v_aliases_k is set");
  } else {
    if (v_new == nullptr) return fail(KVD_ERR_INVALID, "v_new must be non-NULL");
    if (!aligned(v_new, 4)) return fail(KVD_ERR_INVALID, "v_new must be 4-byte aligned");
  }
  // the cache tensors follow the decode entry points' rules (q is not used)
  s = check_tensors(p, k_new, k, v, positions, /*need_q16=*/false);
  if (s != KVD_OK) return s;
  kvd::AppendArgs a{};
  a.k_new = k_new;
  a.v_new = p->v_aliases_k ? nullptr : v_new;
  a.positions = positions;
  a.k = const_cast<void*>(k.data);
  a.k_scale = const_cast<void*>(k.scale);
  a.v = p->v_aliases_k ? nullptr : const_cast<void*>(v.data);
  a.v_scale = p->v_aliases_k ? nullptr : const_cast<void*>(v.scale);
  a.B = p->B;
  a.Hkv = p->Hkv;
  a.Dqk = p->Dqk;
  a.Dv = p->Dv;
  a.kvp = p->kvp;
  a.T = (int32_t)tokens(p);
  a.S_max = p->S_max;
  a.kv_format = p->kv_dtype;
  a.v_aliases_k = p->v_aliases_k != 0;
  a.layout = p->layout;
  set_paging(p, &a);
  const hipError_t e = kvd::launch_append_kv(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVD_ERR_HIP, "append launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t kvd_decode_workspace_bytes(const kvd_problem* p) {
  if (check_problem(p) != KVD_OK) return 0;
  return workspace_o_bytes(p) + workspace_lse_bytes(p);
}

int kvd_decode(const kvd_problem* p, const void* q, kvd_kv k, kvd_kv v, const int32_t* seq_lens,
               void* workspace, float* o, float* lse, kvd_stream_t stream) {
  int s = check_problem(p);
  if (s != KVD_OK) return s;
  s = check_tensors(p, q, k, v, seq_lens);
  if (s != KVD_OK) return s;
  if (workspace == nullptr || !aligned(workspace, 16))
    return fail(KVD_ERR_INVALID, "workspace must be non-NULL and 16-byte aligned");
  float* o_part = static_cast<float*>(workspace);
  float* lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + workspace_o_bytes(p));
  const int64_t rows = (int64_t)p->B * tokens(p) * p->Hq;
  s = check_merge(p->kvp, rows, p->Dv, o_part, lse_part, o, lse);
  if (s != KVD_OK) return s;
  // validate the kernel choice before enqueueing anything
  {
    const kvd::PartialArgs a = make_args(p, q, k, v, seq_lens, o_part, lse_part);
    if (choose(a) == Path::kNone)
      return fail(KVD_ERR_UNSUPPORTED,
                  "no kernel for Hq=%d Hkv=%d Dqk=%d Dv=%d kv_dtype=%d q_dtype=%d v_aliases_k=%d",
                  p->Hq, p->Hkv, p->Dqk, p->Dv, p->kv_dtype, p->q_dtype, p->v_aliases_k);
  }
  s = launch_partial(p, q, k, v, seq_lens, o_part, lse_part, reinterpret_cast<hipStream_t>(stream));
  if (s != KVD_OK) return s;
  return kvd_lse_merge(p->kvp, rows, p->Dv, o_part, lse_part, o, lse, stream);
}

int kvd_decode_noalloc(const kvd_problem* p, const void* q, kvd_kv k, kvd_kv v, const int32_t* seq_lens,
                       float* o, float* lse, kvd_stream_t stream) {
  int s = check_problem(p);
  if (s != KVD_OK) return s;
  s = check_tensors(p, q, k, v, seq_lens);
  if (s != KVD_OK) return s;
  const size_t need = workspace_o_bytes(p) + workspace_lse_bytes(p);
  if (need > (size_t)KVD_NOALLOC_SCRATCH_BYTES)
    return fail(KVD_ERR_UNSUPPORTED,
                "kvd_decode_noalloc: the shard partials need %zu bytes, more than its %zu-byte static array "
                "(kvp*B*q_tokens*Hq*(Dv+1) floats); use kvd_decode with a workspace",
                need, (size_t)KVD_NOALLOC_SCRATCH_BYTES);
  void* ws = noalloc_scratch(&s);
  if (ws == nullptr) return s;
  // from here on exactly kvd_decode with the static array as its workspace
  return kvd_decode(p, q, k, v, seq_lens, ws, o, lse, stream);
}

}  // extern "C"
