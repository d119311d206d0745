/*
 * layer_demo.c — a plain C program that runs one CSA layer and one HCA layer
 * forward through the library's C ABI (include/csa_hip.h), with no Python in
 * the loop: it allocates and copies with the HIP runtime, sizes workspaces with
 * the *_workspace_size() queries and calls the entry points in the order a
 * layer uses them (cf-1.com write-up §3.1–§3.3):
 *
 *   CSA: csa_compress (KV streams) -> csa_compress (indexer key streams)
 *        -> indexer_topk (float32 operands) -> sparse_attn_fwd
 *   HCA: hca_compress -> dense_compressed_attn_fwd
 *
 * Usage:
 *   layer_demo validate
 *       host-side checks only (no device memory, no launch): status strings,
 *       the version string, and calls that must fail validation with the
 *       documented status and a non-empty csa_last_error().
 *   layer_demo run DIR T H H_I D_I K WINDOW
 *       reads float32 inputs from DIR (raw little-endian files written by the
 *       test), runs both layers on one prefill sequence of T tokens (positions
 *       0..T-1, ratio 4 and 128, width 128), and writes the results to DIR.
 *
 * Exit status 0 on success; any failure prints the call, its status and the
 * library's detail, and exits 1.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "csa_hip.h"

#define D 128

static int fail(const char* what, int st) {
  fprintf(stderr, "%s: status %d (%s): %s\n", what, st, csa_status_string(st), csa_last_error());
  return 1;
}

#define HIP_OK(call)                                                             \
  do {                                                                           \
    hipError_t e_ = (call);                                                      \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                 \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

#define CSA_OK_OR_FAIL(call)                                                     \
  do {                                                                           \
    csa_status s_ = (call);                                                      \
    if (s_ != CSA_OK) return fail(#call, (int)s_);                               \
  } while (0)

/* expect a validation failure with the given status and a detail message */
static int expect(const char* what, csa_status got, csa_status want) {
  if (got != want) {
    fprintf(stderr, "%s: got status %d, want %d\n", what, (int)got, (int)want);
    return 1;
  }
  if (csa_last_error()[0] == '\0') {
    fprintf(stderr, "%s: no detail in csa_last_error()\n", what);
    return 1;
  }
  return 0;
}

static int validate(void) {
  int bad = 0;
  if (strcmp(csa_status_string(CSA_OK), "") == 0 || csa_version()[0] == '\0') {
    fprintf(stderr, "empty status or version string\n");
    return 1;
  }
  /* every pointer NULL: rejected before anything touches the device */
  bad |= expect("csa_compress(NULL)",
                csa_compress(NULL, NULL, NULL, NULL, CSA_F32, 1, 64, D, 4, NULL, CSA_F32, NULL, NULL),
                CSA_ERR_NULL);
  bad |= expect("hca_compress(NULL)", hca_compress(NULL, NULL, CSA_F32, 1, 256, D, 128, NULL, CSA_F32, NULL),
                CSA_ERR_NULL);
  bad |= expect("indexer_topk(NULL)",
                indexer_topk(NULL, NULL, NULL, NULL, NULL, CSA_F32, NULL, 1, 16, 4, 4, 64, 4, 8, NULL, NULL, NULL,
                             0, NULL),
                CSA_ERR_NULL);
  bad |= expect("sparse_attn_fwd(NULL)",
                sparse_attn_fwd(NULL, NULL, NULL, NULL, NULL, NULL, NULL, CSA_F32, 1, 16, 4, 16, 16, D, 8, 128, 1.f,
                                NULL, NULL, NULL, 0, 0, NULL),
                CSA_ERR_NULL);
  bad |= expect("dense_compressed_attn_fwd(NULL)",
                dense_compressed_attn_fwd(NULL, NULL, NULL, NULL, NULL, NULL, CSA_F32, 1, 16, 4, 16, 16, D, 4, 128,
                                          1.f, NULL, NULL, NULL, 0, 0, NULL),
                CSA_ERR_NULL);
  if (bad) return 1;
  printf("validate ok (%s)\n", csa_version());
  return 0;
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    return NULL;
  }
  void* p = malloc(bytes ? bytes : 1);
  const size_t got = p ? fread(p, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    fprintf(stderr, "%s: read %zu of %zu bytes\n", path, got, bytes);
    free(p);
    return NULL;
  }
  return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", path);
    if (f) fclose(f);
    return 1;
  }
  fclose(f);
  return 0;
}

/* host file -> new device buffer */
static int upload(const char* dir, const char* name, size_t bytes, void** dev) {
  void* h = read_file(dir, name, bytes);
  if (!h) return 1;
  hipError_t e = hipMalloc(dev, bytes);
  if (e == hipSuccess) e = hipMemcpy(*dev, h, bytes, hipMemcpyHostToDevice);
  free(h);
  if (e != hipSuccess) {
    fprintf(stderr, "upload %s: %s\n", name, hipGetErrorString(e));
    return 1;
  }
  return 0;
}

/* device buffer -> file */
static int download(const char* dir, const char* name, const void* dev, size_t bytes) {
  void* h = malloc(bytes ? bytes : 1);
  if (!h) return 1;
  hipError_t e = hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost);
  int r = e != hipSuccess ? (fprintf(stderr, "download %s: %s\n", name, hipGetErrorString(e)), 1)
                          : write_file(dir, name, h, bytes);
  free(h);
  return r;
}

static int run(const char* dir, int64_t T, int H, int H_I, int d_I, int k, int window) {
  const int64_t N = T / 4, NH = T / 128;
  const size_t f = sizeof(float);
  void *c_a, *c_b, *z_a, *z_b, *ci_a, *ci_b, *zi_a, *zi_b, *q_i, *w, *q, *sink, *c, *z, *q2, *sink2;
  if (upload(dir, "c_a.f32", T * D * f, &c_a) || upload(dir, "c_b.f32", T * D * f, &c_b) ||
      upload(dir, "z_a.f32", T * D * f, &z_a) || upload(dir, "z_b.f32", T * D * f, &z_b) ||
      upload(dir, "ci_a.f32", T * d_I * f, &ci_a) || upload(dir, "ci_b.f32", T * d_I * f, &ci_b) ||
      upload(dir, "zi_a.f32", T * d_I * f, &zi_a) || upload(dir, "zi_b.f32", T * d_I * f, &zi_b) ||
      upload(dir, "q_i.f32", T * H_I * d_I * f, &q_i) || upload(dir, "w.f32", T * H_I * f, &w) ||
      upload(dir, "q.f32", T * H * D * f, &q) || upload(dir, "sink.f32", H * f, &sink) ||
      upload(dir, "c.f32", T * D * f, &c) || upload(dir, "z.f32", T * D * f, &z) ||
      upload(dir, "q2.f32", T * H * D * f, &q2) || upload(dir, "sink2.f32", H * f, &sink2))
    return 1;

  /* positions 0..T-1 and the window rows' first position (0) */
  int32_t* pos_h = (int32_t*)malloc(T * sizeof(int32_t));
  if (!pos_h) return 1;
  for (int64_t t = 0; t < T; ++t) pos_h[t] = (int32_t)t;
  const int32_t zero = 0;
  void *q_pos, *win0;
  HIP_OK(hipMalloc(&q_pos, T * sizeof(int32_t)));
  HIP_OK(hipMemcpy(q_pos, pos_h, T * sizeof(int32_t), hipMemcpyHostToDevice));
  HIP_OK(hipMalloc(&win0, sizeof(int32_t)));
  HIP_OK(hipMemcpy(win0, &zero, sizeof(int32_t), hipMemcpyHostToDevice));
  free(pos_h);

  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));

  /* ---- CSA layer */
  void *kv, *k_i, *idx, *scores, *o, *lse;
  HIP_OK(hipMalloc(&kv, N * D * f));
  HIP_OK(hipMalloc(&k_i, N * d_I * f));
  HIP_OK(hipMalloc(&idx, T * k * sizeof(int32_t)));
  HIP_OK(hipMalloc(&scores, T * N * f));
  HIP_OK(hipMemset(scores, 0, T * N * f));   /* entries past n(p) are left untouched */
  HIP_OK(hipMalloc(&o, T * H * D * f));
  HIP_OK(hipMalloc(&lse, T * H * f));
  CSA_OK_OR_FAIL(csa_compress(c_a, c_b, z_a, z_b, CSA_F32, 1, T, D, 4, kv, CSA_F32, NULL, s));
  CSA_OK_OR_FAIL(csa_compress(ci_a, ci_b, zi_a, zi_b, CSA_F32, 1, T, d_I, 4, k_i, CSA_F32, NULL, s));
  const size_t ws_i = indexer_topk_workspace_size(1, T, N, H_I, d_I, k, CSA_F32);
  void* wsp_i = NULL;
  if (ws_i) HIP_OK(hipMalloc(&wsp_i, ws_i));
  CSA_OK_OR_FAIL(indexer_topk(q_i, NULL, (const float*)w, k_i, NULL, CSA_F32, (const int32_t*)q_pos, 1, T, N, H_I,
                              d_I, 4, k, (int32_t*)idx, (float*)scores, wsp_i, ws_i, s));
  const size_t ws_s = sparse_attn_workspace_size(1, T, H, D, k, window, 0);
  void* wsp_s = NULL;
  if (ws_s) HIP_OK(hipMalloc(&wsp_s, ws_s));
  CSA_OK_OR_FAIL(sparse_attn_fwd(q, kv, (const int32_t*)idx, c_a, (const int32_t*)win0, (const float*)sink,
                                 (const int32_t*)q_pos, CSA_F32, 1, T, N, T, H, D, k, window, 1.0f, o, (float*)lse,
                                 wsp_s, ws_s, 0, s));

  /* ---- HCA layer */
  void *kvh, *o2, *lse2;
  HIP_OK(hipMalloc(&kvh, (NH > 0 ? NH : 1) * D * f));
  HIP_OK(hipMalloc(&o2, T * H * D * f));
  HIP_OK(hipMalloc(&lse2, T * H * f));
  CSA_OK_OR_FAIL(hca_compress(c, z, CSA_F32, 1, T, D, 128, kvh, CSA_F32, s));
  const size_t ws_d = dense_attn_workspace_size(1, T, NH, H, D, window, 0);
  void* wsp_d = NULL;
  if (ws_d) HIP_OK(hipMalloc(&wsp_d, ws_d));
  CSA_OK_OR_FAIL(dense_compressed_attn_fwd(q2, kvh, c, (const int32_t*)win0, (const float*)sink2,
                                           (const int32_t*)q_pos, CSA_F32, 1, T, NH, T, H, D, 128, window, 1.0f, o2,
                                           (float*)lse2, wsp_d, ws_d, 0, s));
  HIP_OK(hipStreamSynchronize(s));

  if (download(dir, "kv.out", kv, N * D * f) || download(dir, "k_i.out", k_i, N * d_I * f) ||
      download(dir, "idx.out", idx, T * k * sizeof(int32_t)) || download(dir, "scores.out", scores, T * N * f) ||
      download(dir, "o.out", o, T * H * D * f) || download(dir, "lse.out", lse, T * H * f) ||
      download(dir, "kvh.out", kvh, NH * D * f) || download(dir, "o2.out", o2, T * H * D * f) ||
      download(dir, "lse2.out", lse2, T * H * f))
    return 1;
  void* bufs[] = {c_a, c_b, z_a, z_b, ci_a, ci_b, zi_a, zi_b, q_i, w, q, sink, c, z, q2, sink2,
                  q_pos, win0, kv, k_i, idx, scores, o, lse, kvh, o2, lse2, wsp_i, wsp_s, wsp_d};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i)
    if (bufs[i]) HIP_OK(hipFree(bufs[i]));
  HIP_OK(hipStreamDestroy(s));
  printf("run ok: T=%lld H=%d H_I=%d d_I=%d k=%d window=%d\n", (long long)T, H, H_I, d_I, k, window);
  return 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "validate") == 0) return validate();
  if (argc == 9 && strcmp(argv[1], "run") == 0) {
    const int64_t T = atoll(argv[3]);
    const int H = atoi(argv[4]), H_I = atoi(argv[5]), d_I = atoi(argv[6]), k = atoi(argv[7]),
              window = atoi(argv[8]);
    if (T < 128 || T % 128 != 0 || H < 16 || H % 16 != 0 || H_I < 1 || (d_I != 64 && d_I != 128) || k < 1 ||
        window < 0) {
      fprintf(stderr, "bad sizes\n");
      return 2;
    }
    return run(argv[2], T, H, H_I, d_I, k, window);
  }
  fprintf(stderr, "usage: %s validate | run DIR T H H_I D_I K WINDOW\n", argv[0]);
  return 2;
}
