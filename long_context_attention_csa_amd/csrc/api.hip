// C ABI of libcsa_hip: argument validation, workspace sizing, status strings,
// kernel timer, and dispatch to the kernels. Contract: include/csa_hip.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "common.hpp"

namespace csa {
hipError_t launch_csa_compress(const void*, const void*, const void*, const void*, csa_dtype, int64_t, int64_t, int,
                               int, void*, csa_dtype, void*, hipStream_t);
hipError_t launch_hca_compress(const void*, const void*, csa_dtype, int64_t, int64_t, int, int, void*, csa_dtype,
                               hipStream_t);
hipError_t launch_csa_append(const void*, const void*, const void*, const void*, csa_dtype, int64_t, int, int,
                             const int32_t*, void*, int64_t, void*, csa_dtype, void*, hipStream_t);
hipError_t launch_hca_append(const void*, const void*, csa_dtype, int64_t, int, int, const int32_t*, void*, int64_t,
                             void*, csa_dtype, hipStream_t);
hipError_t launch_quantize_rows(const void*, csa_dtype, int64_t, int, void*, csa_dtype, void*, hipStream_t);
size_t indexer_ws_bytes(int64_t B, int64_t Tq, int64_t N, int sbytes);
hipError_t launch_indexer_topk(const void*, const void*, const float*, const void*, const void*, csa_dtype,
                               const int32_t*, int64_t, int64_t, int64_t, int, int, int, int, int32_t*, void*, bool,
                               void*, hipStream_t);
size_t attn_ws_bytes(int64_t B, int64_t Tq, int H, int64_t nk_max);
size_t attn_bwd_ws_bytes(bool sparse, int64_t B, int64_t Tq, int64_t N, int64_t T_win, int H, int k, int window);
hipError_t launch_attn_bwd(bool sparse, const void* q, const void* kv, const int32_t* idx, const void* x_win,
                           const int32_t* win_start, const float* sink, const int32_t* q_pos, const void* out,
                           const float* lse, const void* dout, int64_t B, int64_t Tq, int64_t N, int64_t T_win,
                           int H, int k, int window, int ratio, float scale, void* dq, float* dkv, float* dx_win,
                           float* dsink, void* ws, hipStream_t s);
void set_batch_invariant(int on);
int batch_invariant();
hipError_t launch_window_append(const void* x_new, csa_dtype t, int64_t B, const int32_t* pos, void* ring,
                                int64_t R, hipStream_t s);
hipError_t launch_attention(bool sparse, csa_dtype t, const void* q, const void* kv, const int32_t* idx,
                            const void* x_win, const int32_t* win_start, const float* sink, const int32_t* q_pos,
                            int64_t B, int64_t Tq, int64_t N, int64_t T_win, int ring, int H, int k, int window,
                            int ratio, float scale, void* out, float* lse, void* ws, int64_t nk_max, hipStream_t st);

// ------------------------------------------------------------------ kernel timer
namespace {
constexpr int kMaxTimed = 4096;
struct Timer {
  int kid = 0;
  int cap = 0;
  int n = 0;
  hipEvent_t ev[2 * kMaxTimed];
  bool created = false;
} g_timer;
}  // namespace

void timer_before(int kid, hipStream_t s) {
  if (g_timer.kid == kid && g_timer.n < g_timer.cap) (void)hipEventRecord(g_timer.ev[2 * g_timer.n], s);
}
void timer_after(int kid, hipStream_t s) {
  if (g_timer.kid == kid && g_timer.n < g_timer.cap) {
    (void)hipEventRecord(g_timer.ev[2 * g_timer.n + 1], s);
    ++g_timer.n;
  }
}
}  // namespace csa

using namespace csa;

static thread_local std::string g_last_error;

static csa_status fail(csa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
static csa_status fail(csa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

static csa_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return CSA_OK;
  return fail(CSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

static bool is_float(csa_dtype t) { return t == CSA_F32 || t == CSA_BF16; }
static bool is_dtype(int t) { return t >= CSA_F32 && t <= CSA_FP4_E2M1; }

#define CSA_REQUIRE(cond, st, ...) \
  do {                             \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

extern "C" {

const char* csa_status_string(int status) {
  switch (status) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_NULL: return "CSA_ERR_NULL";
    case CSA_ERR_SHAPE: return "CSA_ERR_SHAPE";
    case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED";
    case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE";
    case CSA_ERR_HIP: return "CSA_ERR_HIP";
    default: return "CSA_ERR_UNKNOWN";
  }
}

const char* csa_last_error(void) { return g_last_error.c_str(); }

const char* csa_version(void) { return "csa_hip 0.1 gfx950"; }

csa_status csa_quantize_rows(const void* x, csa_dtype in_t, int64_t rows, int32_t width, void* out, csa_dtype out_t,
                             void* scale, void* stream) {
  g_last_error.clear();
  CSA_REQUIRE(is_dtype(in_t) && is_dtype(out_t), CSA_ERR_UNSUPPORTED, "csa_quantize_rows: unknown dtype");
  CSA_REQUIRE(is_float(in_t), CSA_ERR_UNSUPPORTED, "csa_quantize_rows: input must be CSA_F32 or CSA_BF16");
  CSA_REQUIRE(out_t == CSA_FP8_E4M3 || out_t == CSA_FP4_E2M1, CSA_ERR_UNSUPPORTED,
              "csa_quantize_rows: output must be CSA_FP8_E4M3 or CSA_FP4_E2M1");
  CSA_REQUIRE(rows >= 0 && width > 0 && width <= 4096, CSA_ERR_SHAPE, "csa_quantize_rows: rows=%lld width=%d",
              (long long)rows, width);
  CSA_REQUIRE(width % (out_t == CSA_FP4_E2M1 ? 32 : 8) == 0, CSA_ERR_SHAPE,
              "csa_quantize_rows: width %d must be a multiple of %d", width, out_t == CSA_FP4_E2M1 ? 32 : 8);
  if (rows == 0) return CSA_OK;
  CSA_REQUIRE(x && out && scale, CSA_ERR_NULL, "csa_quantize_rows: x, out and scale are required");
  return hip_status(launch_quantize_rows(x, in_t, rows, width, out, out_t, scale, (hipStream_t)stream),
                    "csa_quantize_rows");
}

csa_status csa_compress(const void* c_a, const void* c_b, const void* z_a, const void* z_b, csa_dtype in_t,
                        int64_t B, int64_t T, int32_t width, int32_t ratio, void* out, csa_dtype out_t,
                        void* out_scale, void* stream) {
  g_last_error.clear();
  CSA_REQUIRE(is_dtype(in_t) && is_dtype(out_t), CSA_ERR_UNSUPPORTED, "csa_compress: unknown dtype");
  CSA_REQUIRE(is_float(in_t), CSA_ERR_UNSUPPORTED, "csa_compress: input must be CSA_F32 or CSA_BF16");
  CSA_REQUIRE(B >= 0 && T >= 0, CSA_ERR_SHAPE, "csa_compress: B=%lld T=%lld", (long long)B, (long long)T);
  CSA_REQUIRE(width == 64 || width == 128, CSA_ERR_UNSUPPORTED, "csa_compress: width %d (64 or 128)", width);
  CSA_REQUIRE(ratio >= 1 && ratio <= 128, CSA_ERR_SHAPE, "csa_compress: ratio %d (1..128)", ratio);
  if (is_float(out_t))
    CSA_REQUIRE(out_scale == nullptr, CSA_ERR_SHAPE, "csa_compress: out_scale must be NULL for a float output");
  const int64_t N = T / ratio;
  if (B * N == 0) return CSA_OK;
  CSA_REQUIRE(c_a && c_b && z_a && z_b && out, CSA_ERR_NULL, "csa_compress: NULL tensor");
  CSA_REQUIRE(is_float(out_t) || out_scale, CSA_ERR_NULL, "csa_compress: out_scale required for %s output",
              out_t == CSA_FP8_E4M3 ? "fp8" : "fp4");
  return hip_status(launch_csa_compress(c_a, c_b, z_a, z_b, in_t, B, T, width, ratio, out, out_t, out_scale,
                                        (hipStream_t)stream),
                    "csa_compress");
}

csa_status hca_compress(const void* c, const void* z, csa_dtype in_t, int64_t B, int64_t T, int32_t width,
                        int32_t ratio, void* out, csa_dtype out_t, void* stream) {
  g_last_error.clear();
  CSA_REQUIRE(is_dtype(in_t) && is_dtype(out_t), CSA_ERR_UNSUPPORTED, "hca_compress: unknown dtype");
  CSA_REQUIRE(is_float(in_t) && is_float(out_t), CSA_ERR_UNSUPPORTED,
              "hca_compress: input and output must be CSA_F32 or CSA_BF16");
  CSA_REQUIRE(B >= 0 && T >= 0, CSA_ERR_SHAPE, "hca_compress: B=%lld T=%lld", (long long)B, (long long)T);
  CSA_REQUIRE(width == 64 || width == 128, CSA_ERR_UNSUPPORTED, "hca_compress: width %d (64 or 128)", width);
  CSA_REQUIRE(ratio >= 1 && ratio <= 4096, CSA_ERR_SHAPE, "hca_compress: ratio %d (1..4096)", ratio);
  const int64_t N = T / ratio;
  if (B * N == 0) return CSA_OK;
  CSA_REQUIRE(c && z && out, CSA_ERR_NULL, "hca_compress: NULL tensor");
  return hip_status(launch_hca_compress(c, z, in_t, B, T, width, ratio, out, out_t, (hipStream_t)stream),
                    "hca_compress");
}

csa_status csa_compress_append(const void* c_a, const void* c_b, const void* z_a, const void* z_b,
                               csa_dtype in_t, int64_t B, int32_t width, int32_t ratio, const int32_t* pos,
                               void* state, int64_t N_cap, void* out, csa_dtype out_t, void* out_scale,
                               void* stream) {
  g_last_error.clear();
  CSA_REQUIRE(is_dtype(in_t) && is_dtype(out_t), CSA_ERR_UNSUPPORTED, "csa_compress_append: unknown dtype");
  CSA_REQUIRE(is_float(in_t), CSA_ERR_UNSUPPORTED, "csa_compress_append: input must be CSA_F32 or CSA_BF16");
  CSA_REQUIRE(B >= 0 && N_cap >= 0, CSA_ERR_SHAPE, "csa_compress_append: B=%lld N_cap=%lld", (long long)B,
              (long long)N_cap);
  CSA_REQUIRE(B <= INT32_MAX, CSA_ERR_SHAPE, "csa_compress_append: B=%lld (< 2^31)", (long long)B);
  CSA_REQUIRE(width == 64 || width == 128, CSA_ERR_UNSUPPORTED, "csa_compress_append: width %d (64 or 128)", width);
  CSA_REQUIRE(ratio >= 1 && ratio <= 128, CSA_ERR_SHAPE, "csa_compress_append: ratio %d (1..128)", ratio);
  if (is_float(out_t))
    CSA_REQUIRE(out_scale == nullptr, CSA_ERR_SHAPE, "csa_compress_append: out_scale must be NULL for a float output");
  if (B == 0) return CSA_OK;
  CSA_REQUIRE(c_a && c_b && z_a && z_b && pos && state && out, CSA_ERR_NULL, "csa_compress_append: NULL tensor");
  CSA_REQUIRE(is_float(out_t) || out_scale, CSA_ERR_NULL, "csa_compress_append: out_scale required for %s output",
              out_t == CSA_FP8_E4M3 ? "fp8" : "fp4");
  return hip_status(launch_csa_append(c_a, c_b, z_a, z_b, in_t, B, width, ratio, pos, state, N_cap, out, out_t,
                                      out_scale, (hipStream_t)stream),
                    "csa_compress_append");
}

csa_status hca_compress_append(const void* c, const void* z, csa_dtype in_t, int64_t B, int32_t width,
                               int32_t ratio, const int32_t* pos, void* state, int64_t N_cap, void* out,
                               csa_dtype out_t, void* stream) {
  g_last_error.clear();
  CSA_REQUIRE(is_dtype(in_t) && is_dtype(out_t), CSA_ERR_UNSUPPORTED, "hca_compress_append: unknown dtype");
  CSA_REQUIRE(is_float(in_t) && is_float(out_t), CSA_ERR_UNSUPPORTED,
              "hca_compress_append: input and output must be CSA_F32 or CSA_BF16");
  CSA_REQUIRE(B >= 0 && N_cap >= 0, CSA_ERR_SHAPE, "hca_compress_append: B=%lld N_cap=%lld", (long long)B,
              (long long)N_cap);
  CSA_REQUIRE(B <= INT32_MAX, CSA_ERR_SHAPE, "hca_compress_append: B=%lld (< 2^31)", (long long)B);
  CSA_REQUIRE(width == 64 || width == 128, CSA_ERR_UNSUPPORTED, "hca_compress_append: width %d (64 or 128)", width);
  CSA_REQUIRE(ratio >= 1 && ratio <= 4096, CSA_ERR_SHAPE, "hca_compress_append: ratio %d (1..4096)", ratio);
  if (B == 0) return CSA_OK;
  CSA_REQUIRE(c && z && pos && state && out, CSA_ERR_NULL, "hca_compress_append: NULL tensor");
  return hip_status(launch_hca_append(c, z, in_t, B, width, ratio, pos, state, N_cap, out, out_t,
                                      (hipStream_t)stream),
                    "hca_compress_append");
}

csa_status csa_set_batch_invariant(int32_t on) {
  g_last_error.clear();
  set_batch_invariant(on);
  return CSA_OK;
}

int32_t csa_get_batch_invariant(void) { return batch_invariant(); }

size_t indexer_topk_workspace_size(int64_t B, int64_t Tq, int64_t N, int32_t H_I, int32_t d_I, int32_t k,
                                   csa_dtype qk_t) {
  (void)H_I; (void)d_I; (void)k; (void)qk_t;
  if (B <= 0 || Tq <= 0 || N < 0) return 0;
  return indexer_ws_bytes(B, Tq, N, 4);
}

size_t indexer_topk_bf16_scores_workspace_size(int64_t B, int64_t Tq, int64_t N, int32_t H_I, int32_t d_I,
                                               int32_t k, csa_dtype qk_t) {
  (void)H_I; (void)d_I; (void)k; (void)qk_t;
  if (B <= 0 || Tq <= 0 || N < 0) return 0;
  return indexer_ws_bytes(B, Tq, N, 2);
}

static csa_status indexer_common(const char* fn, const void* q_idx, const void* q_scale, const float* w,
                                 const void* k_idx, const void* k_scale, csa_dtype qk_t, const int32_t* q_pos,
                                 int64_t B, int64_t Tq, int64_t N, int32_t H_I, int32_t d_I, int32_t ratio, int32_t k,
                                 int32_t* idx_out, void* score_out, bool bf16, void* ws, size_t ws_bytes,
                                 void* stream) {
  CSA_REQUIRE(is_dtype(qk_t), CSA_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, (int)qk_t);
  CSA_REQUIRE(B >= 0 && Tq >= 0 && N >= 0 && N < (int64_t(1) << 30) && B * Tq < (int64_t(1) << 31), CSA_ERR_SHAPE,
              "%s: B=%lld Tq=%lld N=%lld", fn, (long long)B, (long long)Tq, (long long)N);
  CSA_REQUIRE(H_I >= 1 && H_I <= 64, CSA_ERR_UNSUPPORTED, "%s: H_I %d (1..64)", fn, H_I);
  CSA_REQUIRE(d_I == 64 || d_I == 128, CSA_ERR_UNSUPPORTED, "%s: d_I %d (64 or 128)", fn, d_I);
  CSA_REQUIRE(k >= 1 && k <= 2048, CSA_ERR_SHAPE, "%s: k %d (1..2048)", fn, k);
  CSA_REQUIRE(ratio >= 1, CSA_ERR_SHAPE, "%s: ratio %d", fn, ratio);
  const bool quant = qk_t == CSA_FP8_E4M3 || qk_t == CSA_FP4_E2M1;
  CSA_REQUIRE(quant || (q_scale == nullptr && k_scale == nullptr), CSA_ERR_SHAPE,
              "%s: q_scale/k_scale must be NULL for float operands", fn);
  if (B * Tq == 0) return CSA_OK;
  CSA_REQUIRE(q_idx && w && q_pos && idx_out, CSA_ERR_NULL, "%s: NULL tensor", fn);
  CSA_REQUIRE(N == 0 || k_idx, CSA_ERR_NULL, "%s: k_idx is NULL", fn);
  CSA_REQUIRE(!quant || (q_scale && (N == 0 || k_scale)), CSA_ERR_NULL, "%s: scales required", fn);
  CSA_REQUIRE(((uintptr_t)q_idx & 15) == 0 && ((uintptr_t)k_idx & 15) == 0 && ((uintptr_t)k_scale & 3) == 0,
              CSA_ERR_SHAPE, "%s: q_idx and k_idx must be 16-byte aligned, k_scale 4-byte aligned", fn);
  const size_t need = bf16 ? indexer_topk_bf16_scores_workspace_size(B, Tq, N, H_I, d_I, k, qk_t)
                           : indexer_topk_workspace_size(B, Tq, N, H_I, d_I, k, qk_t);
  CSA_REQUIRE(ws && ws_bytes >= need, CSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  return hip_status(launch_indexer_topk(q_idx, q_scale, w, k_idx, k_scale, qk_t, q_pos, B, Tq, N, H_I, d_I, ratio, k,
                                        idx_out, score_out, bf16, ws, (hipStream_t)stream),
                    fn);
}

csa_status indexer_topk(const void* q_idx, const void* q_scale, const float* w, const void* k_idx,
                        const void* k_scale, csa_dtype qk_t, const int32_t* q_pos, int64_t B, int64_t Tq,
                        int64_t N, int32_t H_I, int32_t d_I, int32_t ratio, int32_t k, int32_t* idx_out,
                        float* score_out, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  return indexer_common("indexer_topk", q_idx, q_scale, w, k_idx, k_scale, qk_t, q_pos, B, Tq, N, H_I, d_I, ratio,
                        k, idx_out, score_out, false, ws, ws_bytes, stream);
}

csa_status indexer_topk_bf16_scores(const void* q_idx, const void* q_scale, const float* w, const void* k_idx,
                                    const void* k_scale, csa_dtype qk_t, const int32_t* q_pos, int64_t B,
                                    int64_t Tq, int64_t N, int32_t H_I, int32_t d_I, int32_t ratio, int32_t k,
                                    int32_t* idx_out, uint16_t* score_out, void* ws, size_t ws_bytes,
                                    void* stream) {
  g_last_error.clear();
  return indexer_common("indexer_topk_bf16_scores", q_idx, q_scale, w, k_idx, k_scale, qk_t, q_pos, B, Tq, N, H_I,
                        d_I, ratio, k, idx_out, score_out, true, ws, ws_bytes, stream);
}

static csa_status check_attn_common(const char* fn, const void* q, const void* kv, const void* x_win,
                                    const int32_t* win_start, const int32_t* q_pos, csa_dtype t, int64_t B,
                                    int64_t Tq, int64_t N, int64_t T_win, int32_t H, int32_t d, int32_t window,
                                    void* out) {
  CSA_REQUIRE(is_dtype(t), CSA_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  CSA_REQUIRE(is_float(t), CSA_ERR_UNSUPPORTED, "%s: dtype must be CSA_F32 or CSA_BF16", fn);
  CSA_REQUIRE(B >= 0 && Tq >= 0 && N >= 0 && T_win >= 0 && window >= 0, CSA_ERR_SHAPE,
              "%s: B=%lld Tq=%lld N=%lld T_win=%lld window=%d", fn, (long long)B, (long long)Tq, (long long)N,
              (long long)T_win, window);
  CSA_REQUIRE(d == 128, CSA_ERR_UNSUPPORTED, "%s: d %d (only 128)", fn, d);
  CSA_REQUIRE(H >= 16 && H <= 256 && H % 16 == 0, CSA_ERR_UNSUPPORTED, "%s: H %d (multiple of 16, <= 256)", fn, H);
  if (B * Tq == 0) return CSA_OK;
  CSA_REQUIRE(B <= INT32_MAX / Tq, CSA_ERR_SHAPE, "%s: B*Tq = %lld x %lld must be < 2^31", fn, (long long)B,
              (long long)Tq);
  CSA_REQUIRE(q && q_pos && win_start && out, CSA_ERR_NULL, "%s: NULL tensor", fn);
  CSA_REQUIRE(N == 0 || kv, CSA_ERR_NULL, "%s: kv is NULL", fn);
  CSA_REQUIRE(T_win == 0 || x_win, CSA_ERR_NULL, "%s: x_win is NULL", fn);
  return CSA_OK;
}

size_t sparse_attn_workspace_size(int64_t B, int64_t Tq, int32_t H, int32_t d, int32_t k, int32_t window) {
  (void)d;
  if (B <= 0 || Tq <= 0 || H <= 0) return 0;
  return attn_ws_bytes(B, Tq, H, (int64_t)k + window);
}

csa_status sparse_attn_fwd(const void* q, const void* kv, const int32_t* idx, const void* x_win,
                           const int32_t* win_start, const float* sink, const int32_t* q_pos, csa_dtype t, int64_t B,
                           int64_t Tq, int64_t N, int64_t T_win, int32_t win_ring, int32_t H, int32_t d, int32_t k,
                           int32_t window, float scale, void* out, float* lse, void* ws, size_t ws_bytes,
                           void* stream) {
  g_last_error.clear();
  csa_status st = check_attn_common("sparse_attn_fwd", q, kv, x_win, win_start, q_pos, t, B, Tq, N, T_win, H, d,
                                    window, out);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(k >= 1 && k <= 4096, CSA_ERR_SHAPE, "sparse_attn_fwd: k %d (1..4096)", k);
  CSA_REQUIRE(win_ring == 0 || win_ring == 1, CSA_ERR_SHAPE, "sparse_attn_fwd: win_ring %d (0 or 1)", win_ring);
  if (B * Tq == 0) return CSA_OK;
  CSA_REQUIRE(idx, CSA_ERR_NULL, "sparse_attn_fwd: idx is NULL");
  const size_t need = sparse_attn_workspace_size(B, Tq, H, d, k, window);
  CSA_REQUIRE(need == 0 || (ws && ws_bytes >= need), CSA_ERR_WORKSPACE, "sparse_attn_fwd: workspace %zu < %zu bytes",
              ws_bytes, need);
  return hip_status(launch_attention(true, t, q, kv, idx, x_win, win_start, sink, q_pos, B, Tq, N, T_win, win_ring, H, k,
                                     window, 1, scale, out, lse, need ? ws : nullptr, (int64_t)k + window,
                                     (hipStream_t)stream),
                    "sparse_attn_fwd");
}

size_t dense_attn_workspace_size(int64_t B, int64_t Tq, int64_t N, int32_t H, int32_t d, int32_t window) {
  (void)d;
  if (B <= 0 || Tq <= 0 || H <= 0) return 0;
  return attn_ws_bytes(B, Tq, H, N + window);
}

csa_status dense_compressed_attn_fwd(const void* q, const void* kv, const void* x_win, const int32_t* win_start,
                                     const float* sink, const int32_t* q_pos, csa_dtype t, int64_t B, int64_t Tq,
                                     int64_t N, int64_t T_win, int32_t win_ring, int32_t H, int32_t d, int32_t ratio,
                                     int32_t window, float scale, void* out, float* lse, void* ws, size_t ws_bytes,
                                     void* stream) {
  g_last_error.clear();
  csa_status st = check_attn_common("dense_compressed_attn_fwd", q, kv, x_win, win_start, q_pos, t, B, Tq, N, T_win,
                                    H, d, window, out);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(ratio >= 1, CSA_ERR_SHAPE, "dense_compressed_attn_fwd: ratio %d", ratio);
  CSA_REQUIRE(win_ring == 0 || win_ring == 1, CSA_ERR_SHAPE, "dense_compressed_attn_fwd: win_ring %d (0 or 1)",
              win_ring);
  if (B * Tq == 0) return CSA_OK;
  const size_t need = dense_attn_workspace_size(B, Tq, N, H, d, window);
  CSA_REQUIRE(need == 0 || (ws && ws_bytes >= need), CSA_ERR_WORKSPACE,
              "dense_compressed_attn_fwd: workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(launch_attention(false, t, q, kv, nullptr, x_win, win_start, sink, q_pos, B, Tq, N, T_win, win_ring, H, 0,
                                     window, ratio, scale, out, lse, need ? ws : nullptr, N + window,
                                     (hipStream_t)stream),
                    "dense_compressed_attn_fwd");
}

csa_status csa_window_append(const void* x_new, csa_dtype t, int64_t B, int32_t d, const int32_t* pos, void* ring,
                             int64_t R, void* stream) {
  g_last_error.clear();
  CSA_REQUIRE(is_dtype(t) && is_float(t), CSA_ERR_UNSUPPORTED, "csa_window_append: dtype must be CSA_F32 or CSA_BF16");
  CSA_REQUIRE(d == 128, CSA_ERR_UNSUPPORTED, "csa_window_append: d %d (only 128)", d);
  CSA_REQUIRE(B >= 0 && R >= 1 && B * R < ((int64_t)1 << 40), CSA_ERR_SHAPE, "csa_window_append: B=%lld R=%lld",
              (long long)B, (long long)R);
  if (B == 0) return CSA_OK;
  CSA_REQUIRE(x_new && pos && ring, CSA_ERR_NULL, "csa_window_append: NULL tensor");
  CSA_REQUIRE(((uintptr_t)x_new & 15) == 0 && ((uintptr_t)ring & 15) == 0, CSA_ERR_SHAPE,
              "csa_window_append: x_new and ring must be 16-byte aligned");
  return hip_status(launch_window_append(x_new, t, B, pos, ring, R, (hipStream_t)stream), "csa_window_append");
}

static csa_status check_attn_bwd(const char* fn, const void* q, const void* kv, const void* x_win,
                                 const int32_t* win_start, const float* sink, const int32_t* q_pos, csa_dtype t,
                                 int64_t B, int64_t Tq, int64_t N, int64_t T_win, int32_t H, int32_t d,
                                 int32_t window, const void* out, const float* lse, const void* dout, void* dq,
                                 float* dkv, float* dx_win, float* dsink) {
  csa_status st = check_attn_common(fn, q, kv, x_win, win_start, q_pos, t, B, Tq, N, T_win, H, d, window,
                                    const_cast<void*>(out));
  if (st != CSA_OK) return st;
  CSA_REQUIRE(t == CSA_BF16, CSA_ERR_UNSUPPORTED, "%s: dtype must be CSA_BF16", fn);
  CSA_REQUIRE(H == 64 || H == 128, CSA_ERR_UNSUPPORTED, "%s: H %d (64 or 128)", fn, H);
  if (B * Tq == 0) return CSA_OK;
  CSA_REQUIRE(lse && dout && dq, CSA_ERR_NULL, "%s: NULL lse, dout or dq", fn);
  CSA_REQUIRE(N == 0 || dkv, CSA_ERR_NULL, "%s: dkv is NULL", fn);
  CSA_REQUIRE(T_win == 0 || dx_win, CSA_ERR_NULL, "%s: dx_win is NULL", fn);
  CSA_REQUIRE(!sink || dsink, CSA_ERR_NULL, "%s: dsink is NULL although sink is given", fn);
  CSA_REQUIRE((int64_t)B * (N + T_win) < (int64_t)1 << 31, CSA_ERR_SHAPE, "%s: B*(N+T_win) must be < 2^31", fn);
  return CSA_OK;
}

size_t sparse_attn_bwd_workspace_size(int64_t B, int64_t Tq, int64_t N, int64_t T_win, int32_t H, int32_t d,
                                      int32_t k, int32_t window) {
  (void)d;
  if (B <= 0 || Tq <= 0 || N < 0 || T_win < 0 || H <= 0 || k < 1 || window < 0) return 0;
  return attn_bwd_ws_bytes(true, B, Tq, N, T_win, H, k, window);
}

csa_status sparse_attn_bwd(const void* q, const void* kv, const int32_t* idx, const void* x_win,
                           const int32_t* win_start, const float* sink, const int32_t* q_pos, csa_dtype t, int64_t B,
                           int64_t Tq, int64_t N, int64_t T_win, int32_t H, int32_t d, int32_t k, int32_t window,
                           float scale, const void* out, const float* lse, const void* dout, void* dq, float* dkv,
                           float* dx_win, float* dsink, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  csa_status st = check_attn_bwd("sparse_attn_bwd", q, kv, x_win, win_start, sink, q_pos, t, B, Tq, N, T_win, H, d,
                                 window, out, lse, dout, dq, dkv, dx_win, dsink);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(k >= 1 && k <= 4096, CSA_ERR_SHAPE, "sparse_attn_bwd: k %d (1..4096)", k);
  if (B * Tq == 0) return CSA_OK;
  CSA_REQUIRE(idx, CSA_ERR_NULL, "sparse_attn_bwd: idx is NULL");
  const size_t need = sparse_attn_bwd_workspace_size(B, Tq, N, T_win, H, d, k, window);
  CSA_REQUIRE(ws && ws_bytes >= need, CSA_ERR_WORKSPACE, "sparse_attn_bwd: workspace %zu < %zu bytes", ws_bytes,
              need);
  return hip_status(launch_attn_bwd(true, q, kv, idx, x_win, win_start, sink, q_pos, out, lse, dout, B, Tq, N, T_win,
                                    H, k, window, 1, scale, dq, dkv, dx_win, dsink, ws, (hipStream_t)stream),
                    "sparse_attn_bwd");
}

size_t dense_attn_bwd_workspace_size(int64_t B, int64_t Tq, int64_t N, int64_t T_win, int32_t H, int32_t d,
                                     int32_t window) {
  (void)d;
  if (B <= 0 || Tq <= 0 || N < 0 || T_win < 0 || H <= 0 || window < 0) return 0;
  return attn_bwd_ws_bytes(false, B, Tq, N, T_win, H, 0, window);
}

csa_status dense_compressed_attn_bwd(const void* q, const void* kv, const void* x_win, const int32_t* win_start,
                                     const float* sink, const int32_t* q_pos, csa_dtype t, int64_t B, int64_t Tq,
                                     int64_t N, int64_t T_win, int32_t H, int32_t d, int32_t ratio, int32_t window,
                                     float scale, const void* out, const float* lse, const void* dout, void* dq,
                                     float* dkv, float* dx_win, float* dsink, void* ws, size_t ws_bytes,
                                     void* stream) {
  g_last_error.clear();
  csa_status st = check_attn_bwd("dense_compressed_attn_bwd", q, kv, x_win, win_start, sink, q_pos, t, B, Tq, N,
                                 T_win, H, d, window, out, lse, dout, dq, dkv, dx_win, dsink);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(ratio >= 1, CSA_ERR_SHAPE, "dense_compressed_attn_bwd: ratio %d", ratio);
  if (B * Tq == 0) return CSA_OK;
  const size_t need = dense_attn_bwd_workspace_size(B, Tq, N, T_win, H, d, window);
  CSA_REQUIRE(ws && ws_bytes >= need, CSA_ERR_WORKSPACE, "dense_compressed_attn_bwd: workspace %zu < %zu bytes",
              ws_bytes, need);
  return hip_status(launch_attn_bwd(false, q, kv, nullptr, x_win, win_start, sink, q_pos, out, lse, dout, B, Tq, N,
                                    T_win, H, 0, window, ratio, scale, dq, dkv, dx_win, dsink, ws,
                                    (hipStream_t)stream),
                    "dense_compressed_attn_bwd");
}

csa_status csa_kernel_timer_start(int32_t kernel_id, int32_t max_launches) {
  g_last_error.clear();
  CSA_REQUIRE(kernel_id >= CSA_KID_COMPRESS && kernel_id <= CSA_KID_ATTN_BWD, CSA_ERR_SHAPE,
              "csa_kernel_timer_start: kernel id %d", kernel_id);
  CSA_REQUIRE(max_launches >= 1 && max_launches <= kMaxTimed, CSA_ERR_SHAPE,
              "csa_kernel_timer_start: max_launches %d (1..%d)", max_launches, kMaxTimed);
  if (!g_timer.created) {
    for (int i = 0; i < 2 * kMaxTimed; ++i) {
      hipError_t e = hipEventCreate(&g_timer.ev[i]);
      if (e != hipSuccess) return hip_status(e, "csa_kernel_timer_start");
    }
    g_timer.created = true;
  }
  g_timer.kid = kernel_id;
  g_timer.cap = max_launches;
  g_timer.n = 0;
  return CSA_OK;
}

int32_t csa_kernel_timer_read(float* ms_out, int32_t capacity) {
  const int n = g_timer.n;
  g_timer.kid = 0;
  g_timer.cap = 0;
  g_timer.n = 0;
  if (n == 0) return 0;
  if (hipEventSynchronize(g_timer.ev[2 * n - 1]) != hipSuccess) return -1;
  for (int i = 0; i < n && i < capacity; ++i) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_timer.ev[2 * i], g_timer.ev[2 * i + 1]) != hipSuccess) return -1;
    ms_out[i] = ms;
  }
  return n;
}

}  // extern "C"
