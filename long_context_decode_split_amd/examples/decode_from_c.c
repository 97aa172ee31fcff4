/*
 * Exact split-KV decode through the C ABI of libkvd.so, from plain C.
 *
 * The caller owns every device buffer: this program allocates them with the
 * HIP runtime, copies the inputs in, asks the library for the workspace size,
 * runs kvd_decode on the null stream and copies o and lse back.
 *
 * Usage: decode_from_c DIR
 *   DIR/problem.txt  "B Hq Hkv Dqk Dv S_max kvp q_dtype kv_dtype q_tokens"
 *                    (dtypes as kvd_dtype codes), contiguous layout
 *   DIR/q.bin, k.bin, v.bin (absent when Dv < Dqk and V aliases K: see below),
 *   k_scale.bin, v_scale.bin (fp8 and MXFP4 only), seq_lens.bin (int32 [B]):
 *                    raw little-endian arrays in the layouts of kvd.h
 *   writes DIR/o.bin (float [B,T,Hq,Dv]) and DIR/lse.bin (float [B,T,Hq]).
 * A missing v.bin means V aliases the first Dv columns of K.
 * Exit status 0 on success; messages go to stderr.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "kvd.h"

static int read_file(const char* dir, const char* name, void** data, size_t* bytes) {
  char path[4096];
  snprintf(path, sizeof(path), "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return 0;
  fseek(f, 0, SEEK_END);
  const long n = ftell(f);
  fseek(f, 0, SEEK_SET);
  *data = malloc(n > 0 ? (size_t)n : 1);
  *bytes = (size_t)n;
  const size_t got = fread(*data, 1, (size_t)n, f);
  fclose(f);
  if (got != (size_t)n) {
    fprintf(stderr, "short read of %s\n", path);
    exit(2);
  }
  return 1;
}

static void write_file(const char* dir, const char* name, const void* data, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof(path), "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(data, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", path);
    exit(2);
  }
  fclose(f);
}

#define HIP_OK(call)                                                      \
  do {                                                                    \
    hipError_t e_ = (call);                                               \
    if (e_ != hipSuccess) {                                               \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));          \
      exit(3);                                                            \
    }                                                                     \
  } while (0)

/* Copy a host file into a new device buffer (NULL if the file is absent). */
static void* upload(const char* dir, const char* name) {
  void* h = NULL;
  size_t n = 0;
  if (!read_file(dir, name, &h, &n)) return NULL;
  void* d = NULL;
  HIP_OK(hipMalloc(&d, n > 0 ? n : 16));
  HIP_OK(hipMemcpy(d, h, n, hipMemcpyHostToDevice));
  free(h);
  return d;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  char path[4096];
  snprintf(path, sizeof(path), "%s/problem.txt", dir);
  FILE* f = fopen(path, "r");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    return 2;
  }
  kvd_problem p;
  memset(&p, 0, sizeof(p));
  long long s_max = 0;
  if (fscanf(f, "%d %d %d %d %d %lld %d %d %d %d", &p.B, &p.Hq, &p.Hkv, &p.Dqk, &p.Dv, &s_max, &p.kvp,
             &p.q_dtype, &p.kv_dtype, &p.q_tokens) != 10) {
    fprintf(stderr, "malformed %s\n", path);
    return 2;
  }
  fclose(f);
  p.S_max = s_max;
  p.layout = KVD_LAYOUT_CONTIGUOUS;

  kvd_kv k = {upload(dir, "k.bin"), upload(dir, "k_scale.bin")};
  kvd_kv v = {upload(dir, "v.bin"), upload(dir, "v_scale.bin")};
  p.v_aliases_k = v.data == NULL;
  void* q = upload(dir, "q.bin");
  int32_t* seq_lens = (int32_t*)upload(dir, "seq_lens.bin");

  const size_t ws_bytes = kvd_decode_workspace_bytes(&p);
  if (ws_bytes == 0) {
    fprintf(stderr, "invalid problem: %s\n", kvd_last_error());
    return 4;
  }
  const int T = p.q_tokens > 0 ? p.q_tokens : 1;
  const size_t rows = (size_t)p.B * T * p.Hq;
  void* ws = NULL;
  float *o = NULL, *lse = NULL;
  HIP_OK(hipMalloc(&ws, ws_bytes));
  HIP_OK(hipMalloc((void**)&o, rows * p.Dv * sizeof(float)));
  HIP_OK(hipMalloc((void**)&lse, rows * sizeof(float)));

  const int status = kvd_decode(&p, q, k, v, seq_lens, ws, o, lse, NULL);
  if (status != KVD_OK) {
    fprintf(stderr, "kvd_decode: %s: %s\n", kvd_status_string(status), kvd_last_error());
    return 5;
  }
  HIP_OK(hipDeviceSynchronize());

  float* ho = (float*)malloc(rows * p.Dv * sizeof(float));
  float* hl = (float*)malloc(rows * sizeof(float));
  HIP_OK(hipMemcpy(ho, o, rows * p.Dv * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hl, lse, rows * sizeof(float), hipMemcpyDeviceToHost));
  write_file(dir, "o.bin", ho, rows * p.Dv * sizeof(float));
  write_file(dir, "lse.bin", hl, rows * sizeof(float));
  fprintf(stderr, "decode_from_c: %zu rows, workspace %zu bytes\n", rows, ws_bytes);

  free(ho);
  free(hl);
  HIP_OK(hipFree(ws));
  HIP_OK(hipFree(o));
  HIP_OK(hipFree(lse));
  HIP_OK(hipFree(q));
  HIP_OK(hipFree(seq_lens));
  HIP_OK(hipFree((void*)k.data));
  if (k.scale) HIP_OK(hipFree((void*)k.scale));
  if (v.data) HIP_OK(hipFree((void*)v.data));
  if (v.scale) HIP_OK(hipFree((void*)v.scale));
  return 0;
}
