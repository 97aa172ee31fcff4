/*
 * kvd.h — exact split-KV decode attention on MI355X (gfx950): the C ABI of libkvd.so.
 *
 * The operation.  One new query token per request attends to every cached
 * token of that request: for query head h of request b, with KV head
 * kvh = floor(h / G), G = Hq / Hkv, and L = seq_lens[b],
 *     x_s = sm_scale * <q[b,h,:], k[b,kvh,s,:]>          s = 0 .. L-1
 *     o[b,h,:] = sum_s softmax(x)_s * v[b,kvh,s,:],  lse[b,h] = ln sum_s exp(x_s)
 * i.e. softmax(q K^T / sqrt(d)) V for a single query row (sm_scale defaults to
 * 1/sqrt(Dqk)).  Grouped-query attention maps consecutive query heads onto one
 * KV head; multi-head latent attention is the case Hkv = 1 with V the first Dv
 * columns of the cached latent K.
 *
 * Several query tokens (q_tokens = T > 1).  A turn that brings T new tokens
 * to a request (the pass-Q setting of the "Context Parallelism for Scalable
 * Million-Token Inference" note, section "A runtime heuristic chooses the
 * ring direction": Q is [T, N_H, D_H] while K and V are [T + P, N_KV, D_H],
 * so the new tokens' keys and values are in the cache, appended first) has
 * query token t at position L - T + t, and attention among the new tokens is
 * causal: query t attends to positions 0 .. L - T + t, i.e. the sum over s
 * above stops at L - T + t.  A query with no such position (L < T - t)
 * yields o = 0, lse = -inf.  T = 1 is the single-token decode.
 *
 * The split.  Following KV parallelism in "Helix Parallelism: Why Tensor
 * Parallelism Hits a Wall at Million-Token Context" (section "Sharding the
 * sequence instead"), the sequence of each request is cut into kvp shards;
 * each shard yields its own normalized partial output and the log-sum-exp of
 * its logits, and a log-sum-exp merge of the shards gives the exact
 * full-context result (same article, the merge sketch; and the exact merge
 * equation in the "Context Parallelism for Scalable Million-Token Inference"
 * note, section "Pass-KV keeps queries local and circulates keys and values").
 * Shard j of a request with L tokens covers tokens [j*C, min(L, (j+1)*C)),
 * C = ceil(ceil(L / kvp) / 16) * 16; a shard starting at or past L is empty
 * and yields o = 0, lse = -inf (weight zero in the merge).  Partials are laid
 * out shard-major, so shard j's block is exactly what KV-parallel rank j would
 * send in the all-to-all.
 *
 * Conventions for every entry point:
 *  - Ownership: every pointer argument (except `p`, which is host memory) is a
 *    caller-owned DEVICE pointer.  The library never allocates, frees or
 *    synchronizes; it keeps no state between calls and is reentrant (apart
 *    from raising, once per process and thread-safely, the dynamic-LDS limit
 *    of the kernels that use more than 64 KB of it).
 *  - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL is the null
 *    stream) and the call returns without waiting for it.
 *  - Layouts: contiguous row-major.  q [B,T,Hq,Dqk]; k.data [B,Hkv,S_max,Dqk];
 *    v.data [B,Hkv,S_max,Dv]; seq_lens int32 [B]; outputs are fp32:
 *    o [B,T,Hq,Dv], lse [B,T,Hq] (natural log), o_part [kvp,B,T,Hq,Dv],
 *    lse_part [kvp,B,T,Hq] (T = 1: the [B,Hq,...] arrays of one token).
 *  - KV formats (kv_dtype):
 *      KVD_F32, KVD_BF16: plain elements; scale must be NULL.
 *      KVD_FP8_E4M3: OCP E4M3 ("fn") codes, one byte per element; scale is a
 *        float [B,Hkv] per tensor: element value = code value * scale[b,kvh].
 *      KVD_MXFP4: OCP MXFP4; data rows hold D/2 bytes, element 2i in bits
 *        [3:0] and 2i+1 in bits [7:4] of byte i; scale is uint8 E8M0
 *        [B,Hkv,S_max,D/32], value 2^(E-127) for the 32 contiguous elements
 *        of its block.  Requires D % 32 == 0.
 *  - Alignment: q, k.data, v.data, o, o_part and workspace must be 16-byte
 *    aligned; seq_lens, lse, lse_part and scale pointers 4-byte aligned.
 *  - Errors: every argument is validated on the host before anything is
 *    enqueued; an invalid call returns KVD_ERR_INVALID (malformed) or
 *    KVD_ERR_UNSUPPORTED (well formed, but no kernel of the library handles it)
 *    and enqueues nothing.  A launch failure reported by the HIP runtime
 *    returns KVD_ERR_HIP.  kvd_last_error() gives the calling thread's message
 *    for its last failed call.
 *  - Kernel choice: the library picks the fastest kernel that handles the
 *    problem (matrix-core kernels for 16-head GQA groups and for 576/512
 *    latent heads, the vector-ALU kernel otherwise).  Setting the environment
 *    variable KVD_PATH=valu before the first call restricts it to the
 *    vector-ALU kernel, e.g. to cross-check the two.
 *  - Device-side preconditions: 0 <= seq_lens[b] <= S_max (contiguous
 *    layout) or <= kvp * S_max (sharded layouts).  Kernels clamp each length,
 *    and each shard's length into [0, S_max], so no read ever leaves the
 *    cache.  A request with L = 0 yields o = 0 and lse = -inf.
 *
 * Cache layouts (kvd_problem.layout).  Which shard stores global token
 * position i of a request:
 *  - KVD_LAYOUT_CONTIGUOUS: one cache [B,Hkv,S_max,D]; token i is row i, and
 *    shards are cut at decode time by the split rule above.
 *  - KVD_LAYOUT_STRIPED: token i belongs to shard i mod kvp, at local row
 *    i div kvp (the inference-parallelism survey, sequence layouts section,
 *    "Striped": rank = position mod CP, each rank storing its tokens
 *    compactly).
 *  - KVD_LAYOUT_STAGGERED16: tokens are dealt to shards in runs of 16: token
 *    i belongs to shard (i div 16) mod kvp, at local row
 *    16 * (i div (16 kvp)) + i mod 16 (Helix article, section "Then
 *    reconfigure the same GPUs": new tokens go to one KV-parallel rank for 16
 *    decode steps, then to the next, round-robin).
 *  - KVD_LAYOUT_PAGED: a pool of fixed-size blocks [num_blocks,Hkv,
 *    block_len,D] shared by all requests (the per-rank block cache of the
 *    "Attention DP" design note, section "KV Cache"); block_table
 *    [B,max_blocks] (int32, device) lists each request's blocks in order, so
 *    token i of request b is row i mod block_len of block
 *    block_table[b, i div block_len].  Shards are cut by the split rule over
 *    token positions, as for the contiguous layout.
 * A sharded cache is k.data [kvp,B,Hkv,S_max,Dqk] (v.data likewise; MXFP4
 * scales [kvp,B,Hkv,S_max,D/32]; fp8 scales stay [B,Hkv]): shard j of
 * request b holds its tokens in increasing position at rows 0 .. L_j - 1,
 * and S_max is the capacity of one shard.  A paged cache is k.data
 * [num_blocks,Hkv,block_len,Dqk] (MXFP4 scales [num_blocks,Hkv,block_len,
 * D/32]; fp8 scales stay [B,Hkv]); block_len is a power of two in
 * [16, 2^20], S_max is not used, lengths are clamped to max_blocks *
 * block_len and block ids into [0, num_blocks).  Decode results do not
 * depend on the layout; shard j's partial is attention over the tokens shard
 * j holds (for query token t: those at positions up to L - T + t, which are
 * the first rows of the shard).
 */
#ifndef KVD_H_
#define KVD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVD_ABI_VERSION 5

/* Bytes of the static device array behind kvd_decode_noalloc (96 MiB per
 * device the library runs on). */
#define KVD_NOALLOC_SCRATCH_BYTES (96u * 1024u * 1024u)

typedef enum {
  KVD_OK = 0,
  KVD_ERR_INVALID = 1,
  KVD_ERR_UNSUPPORTED = 2,
  KVD_ERR_HIP = 3
} kvd_status;

typedef enum {
  KVD_F32 = 0,
  KVD_BF16 = 1,
  KVD_FP8_E4M3 = 2,
  KVD_MXFP4 = 3
} kvd_dtype;

typedef enum {
  KVD_LAYOUT_CONTIGUOUS = 0,
  KVD_LAYOUT_STRIPED = 1,
  KVD_LAYOUT_STAGGERED16 = 2,
  KVD_LAYOUT_PAGED = 3
} kvd_layout;

/* A hipStream_t (layout-compatible; NULL is the null stream). */
typedef struct ihipStream_t* kvd_stream_t;

/* Shape of one decode step: B requests, Hq query heads on Hkv KV heads of
 * widths Dqk (q, k) and Dv (v, o), cache stride S_max tokens, kvp shards. */
typedef struct {
  int32_t B;            /* requests, >= 1 */
  int32_t Hq;           /* query heads, >= 1, Hq % Hkv == 0 */
  int32_t Hkv;          /* KV heads, >= 1 */
  int32_t Dqk;          /* q/k head width */
  int32_t Dv;           /* v/o head width (== Dqk except latent attention) */
  int64_t S_max;        /* token stride of the cache (of one shard for the
                           sharded layouts), >= 1 */
  int32_t kvp;          /* shards per request, 1 .. 4096 */
  int32_t q_dtype;      /* kvd_dtype: KVD_F32 or KVD_BF16 */
  int32_t kv_dtype;     /* kvd_dtype of K and V */
  float sm_scale;       /* logit scale, >= 0 and finite; 0 means 1/sqrt(Dqk) */
  int32_t v_aliases_k;  /* nonzero: V is k[..., :Dv] (Dv <= Dqk); v.data and
                           v.scale must be NULL */
  int32_t layout;       /* kvd_layout of the cache; zero-initialized problems
                           are contiguous */
  int32_t block_len;    /* KVD_LAYOUT_PAGED only: tokens per block */
  int32_t max_blocks;   /* KVD_LAYOUT_PAGED only: columns of block_table */
  int64_t num_blocks;   /* KVD_LAYOUT_PAGED only: blocks in the pool */
  const int32_t* block_table;  /* KVD_LAYOUT_PAGED only: device [B,max_blocks] */
  int32_t q_tokens;     /* T, query tokens per request (and new tokens per
                           request for kvd_append_kv), 0 .. 65536; 0 means 1 */
} kvd_problem;

/* One cache tensor: element data and, for fp8 / MXFP4, its scales. */
typedef struct {
  const void* data;
  const void* scale;
} kvd_kv;

/* Shard partials: for every request b, shard j < kvp, query token t and
 * query head h, o_part[j,b,t,h,:] = softmax-weighted mean of V over the tokens
 * of shard j that query t sees (fp32) and lse_part[j,b,t,h] = ln sum of
 * exp(x_s) over them (fp32), i.e. the local output and log-sum-exp that each
 * KV-parallel rank computes over its own slice of the sequence in the Helix
 * article (section "Sharding the sequence instead").  q, the cache tensors
 * and seq_lens are read; o_part [kvp,B,T,Hq,Dv] and lse_part [kvp,B,T,Hq]
 * (device, caller-owned) are written in full, empty shards included (o = 0,
 * lse = -inf).  Errors: KVD_ERR_INVALID for a malformed problem or a NULL /
 * misaligned pointer; KVD_ERR_UNSUPPORTED when no kernel handles the shape. */
int kvd_decode_partial(const kvd_problem* p, const void* q, kvd_kv k, kvd_kv v,
                       const int32_t* seq_lens, float* o_part, float* lse_part,
                       kvd_stream_t stream);

/* Exact log-sum-exp merge of kvp partials for `rows` independent rows: the
 * per-token merge of KV-parallel fragments in the Helix article (section
 * "Sharding the sequence instead": rescale each fragment's output by the
 * exponential of its lse relative to the largest, sum, divide by the summed
 * weights) and the exact merge equation of the pass-KV ring in the "Context
 * Parallelism for Scalable Million-Token Inference" note (section "Pass-KV
 * keeps queries local and circulates keys and values"):
 * M = max_j lse_part[j,r]; w_j = exp(lse_part[j,r] - M) (0 for an empty
 * shard); o[r,:] = sum_j w_j o_part[j,r,:] / sum_j w_j; lse[r] = M + ln sum_j
 * w_j; rows whose shards are all empty give o = 0, lse = -inf.  Shards are
 * summed in ascending j, so results are deterministic.  o_part is
 * [kvp,rows,Dv], lse_part [kvp,rows] (fp32, device); o [rows,Dv], lse [rows]
 * (fp32, device, written); Dv % 4 == 0; rows may be 0 (nothing is enqueued).
 * Errors: KVD_ERR_INVALID for kvp outside [1, 4096], rows < 0, a bad Dv, or a
 * NULL / misaligned pointer when rows > 0. */
int kvd_lse_merge(int32_t kvp, int64_t rows, int32_t Dv, const float* o_part,
                  const float* lse_part, float* o, float* lse, kvd_stream_t stream);

/* Bytes of device workspace kvd_decode needs for problem p (the shard
 * partials, 256-byte aligned pieces); 0 if p is invalid. */
size_t kvd_decode_workspace_bytes(const kvd_problem* p);

/* The whole KV-parallel decode flow of the Helix article (section "Sharding
 * the sequence instead": every KV-parallel rank runs attention over its shard
 * and returns its partial output with the log-sum-exp, and the partials are
 * merged per token into the exact full-context result) on one device:
 * kvd_decode_partial into `workspace` (o_part at its start, lse_part at the
 * next 256-byte boundary after kvp*B*T*Hq*Dv floats; the caller allocates
 * kvd_decode_workspace_bytes(p) device bytes, 16-byte aligned, and owns them)
 * followed by kvd_lse_merge (rows = B*T*Hq) into o [B,T,Hq,Dv] and lse
 * [B,T,Hq], both on `stream`.  The workspace holds intermediate values only;
 * its contents after the call are unspecified.  Validation covers both steps
 * before anything is enqueued (the same errors as kvd_decode_partial). */
int kvd_decode(const kvd_problem* p, const void* q, kvd_kv k, kvd_kv v,
               const int32_t* seq_lens, void* workspace, float* o, float* lse,
               kvd_stream_t stream);

/* kvd_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * shard partials go to a static device array of KVD_NOALLOC_SCRATCH_BYTES
 * that the library holds on each device it runs on, from the first call on
 * that device until the process ends; nothing is allocated or freed by the
 * call.  Arguments, layouts, results and errors are those of kvd_decode
 * without the workspace, plus KVD_ERR_UNSUPPORTED (nothing enqueued) when
 * kvd_decode_workspace_bytes(p) exceeds KVD_NOALLOC_SCRATCH_BYTES.  All calls
 * on one device share that array, and every call overwrites all of the part
 * it uses before reading it (no state carries over between calls); calls
 * whose work can overlap on one device (different streams, or different host
 * threads without ordering) race on it and must be serialized by the caller,
 * e.g. by issuing them on one stream. */
int kvd_decode_noalloc(const kvd_problem* p, const void* q, kvd_kv k, kvd_kv v,
                       const int32_t* seq_lens, float* o, float* lse, kvd_stream_t stream);

/* Append T = q_tokens new tokens per request to the cache (the decode step's
 * KV write, or the new tokens of a multi-token turn).  For every request b,
 * token t and KV head kvh, the fp32 rows k_new[b,t,kvh,:] (Dqk values) and
 * v_new[b,t,kvh,:] (Dv values) are encoded to kv_dtype and stored at global
 * position positions[b] + t under p->layout (contiguous: that row; sharded:
 * the owner shard's local row; paged: the row of the position's block in the
 * block table).  Encodings:
 *   KVD_F32: copied.  KVD_BF16: round to nearest, ties to even.
 *   KVD_FP8_E4M3: y = x / scale[b,kvh] in fp32 (the slab's existing scale,
 *     read, not changed), then the nearest E4M3 value, ties to even,
 *     saturated to +-448.
 *   KVD_MXFP4: per block of 32 elements E = clamp(floor(log2 amax) - 2 + 127,
 *     0, 254) (127 for an all-zero block), written to the row's scale bytes;
 *     each element x * 2^(127 - E) becomes the nearest E2M1 value, ties to
 *     even, saturated to +-6 (OCP MX).
 * k_new [B,T,Hkv,Dqk] and v_new [B,T,Hkv,Dv] are fp32 device arrays of finite
 * values, 4-byte aligned; v_new must be NULL when V aliases K.  positions is
 * an int32 [B] device array; a request whose positions[b] is negative is
 * skipped, and so is each token whose row falls outside the cache
 * (contiguous: >= S_max; sharded: local row >= S_max; paged: position >=
 * max_blocks * block_len or a block id outside [0, num_blocks)).  Tokens of
 * one call must not share a row (positions[b] + t distinct per request).  k and v are the cache tensors of kvd_decode_partial
 * (written through their const pointers).  kvp and layout of p define the
 * map; q_dtype and sm_scale are ignored. */
int kvd_append_kv(const kvd_problem* p, const float* k_new, const float* v_new,
                  const int32_t* positions, kvd_kv k, kvd_kv v, kvd_stream_t stream);

/* Static description of a status code. */
const char* kvd_status_string(int status);

/* Message of the calling thread's last failed call ("" if none). */
const char* kvd_last_error(void);

/* KVD_ABI_VERSION of the library. */
int kvd_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVD_H_ */
