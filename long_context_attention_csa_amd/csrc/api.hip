// C ABI of libcsa_hip: argument validation, workspace sizing, status strings,
// kernel timer, and dispatch to the kernels. Contract: include/csa_hip.h
// (the timer: include/csa_hip_timer.h).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>

#include "../../include/csa_hip_timer.h"
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
size_t indexer_ws_bytes(int64_t B, int64_t Tq, int64_t N, int sbytes, int d_I, csa_dtype fmt, int k);
hipError_t launch_indexer_topk(const void*, const void*, const float*, const void*, const void*, csa_dtype,
                               const int32_t*, int64_t, int64_t, int64_t, int, int, int, int, int32_t*, void*, bool,
                               void*, hipStream_t);
hipError_t launch_indexer_scores(const void*, const void*, const float*, const void*, const void*, csa_dtype,
                                 const int32_t*, int64_t, int64_t, int64_t, int, int, int, float*, hipStream_t);
hipError_t launch_state_checkpoint(const void* state, int64_t B, int64_t seq_bytes, const int32_t* pos, int period,
                                   void* ckpt, int64_t n_slots, hipStream_t s);
hipError_t launch_state_restore(const void* ckpt, int64_t B, int64_t seq_bytes, int64_t n_slots, const int32_t* slot,
                                void* state, hipStream_t s);
hipError_t launch_ring_fill(const void* hist, int64_t B, int64_t T_hist, int64_t row_bytes, const int32_t* pos,
                            int64_t R, void* ring, hipStream_t s);
hipError_t launch_gemm_bf16(const void* A, int64_t lda, int64_t sA, const void* W, int64_t ldw, int64_t sW, void* C,
                            int64_t ldc, int64_t sC, int64_t M, int64_t N, int64_t K, int64_t G, bool out_bf16,
                            hipStream_t s);
size_t attn_ws_bytes(int64_t B, int64_t Tq, int H, int64_t nk_max, bool batch_inv);
size_t attn_bwd_ws_bytes(bool sparse, int64_t B, int64_t Tq, int64_t N, int64_t T_win, int H, int k, int window);
hipError_t launch_attn_bwd(bool sparse, const void* q, const void* kv, const int32_t* idx, const void* x_win,
                           const int32_t* win_start, const float* sink, const int32_t* q_pos, const void* out,
                           const float* lse, const void* dout, int64_t B, int64_t Tq, int64_t N, int64_t T_win,
                           int H, int k, int window, int ratio, float scale, void* dq, float* dkv, float* dx_win,
                           float* dsink, void* ws, hipStream_t s);
hipError_t launch_window_append(const void* x_new, csa_dtype t, int64_t B, const int32_t* pos, void* ring,
                                int64_t R, hipStream_t s);
hipError_t launch_attention(bool sparse, csa_dtype t, const void* q, const void* kv, const int32_t* idx,
                            const void* x_win, const int32_t* win_start, const float* sink, const int32_t* q_pos,
                            int64_t B, int64_t Tq, int64_t N, int64_t T_win, int ring, int H, int k, int window,
                            int ratio, float scale, void* out, float* lse, void* ws, int64_t nk_max, bool batch_inv,
                            hipStream_t st);

// ------------------------------------------------------------------ kernel timer
// Disarmed by default: a launch then costs one relaxed atomic load. Armed, the
// events around each launch of the chosen kernel are recorded under a lock.
namespace {
constexpr int kMaxTimed = 4096;
struct Timer {
  std::mutex mu;
  std::atomic<int> kid{0};
  int cap = 0;
  int n = 0;
  bool open = false;     // a launch's first event is recorded, its second not yet
  hipEvent_t ev[2 * kMaxTimed];
  bool created = false;
} g_timer;
}  // namespace

// The thread that records a launch's first event holds the lock until the
// launch and its second event are enqueued, so the pair brackets that launch.
thread_local bool t_timer_locked = false;

void timer_before(int kid, hipStream_t s) {
  if (g_timer.kid.load(std::memory_order_relaxed) != kid) return;
  g_timer.mu.lock();
  t_timer_locked = true;
  if (g_timer.kid.load() == kid && g_timer.n < g_timer.cap) {
    (void)hipEventRecord(g_timer.ev[2 * g_timer.n], s);
    g_timer.open = true;
  }
}
void timer_after(int, hipStream_t s) {
  if (!t_timer_locked) return;
  if (g_timer.open) {
    (void)hipEventRecord(g_timer.ev[2 * g_timer.n + 1], s);
    ++g_timer.n;
    g_timer.open = false;
  }
  t_timer_locked = false;
  g_timer.mu.unlock();
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
                             void* scale, hipStream_t stream) {
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
  return hip_status(launch_quantize_rows(x, in_t, rows, width, out, out_t, scale, stream),
                    "csa_quantize_rows");
}

csa_status csa_compress(const void* c_a, const void* c_b, const void* z_a, const void* z_b, csa_dtype in_t,
                        int64_t B, int64_t T, int32_t width, int32_t ratio, void* out, csa_dtype out_t,
                        void* out_scale, hipStream_t stream) {
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
                                        stream),
                    "csa_compress");
}

csa_status hca_compress(const void* c, const void* z, csa_dtype in_t, int64_t B, int64_t T, int32_t width,
                        int32_t ratio, void* out, csa_dtype out_t, hipStream_t stream) {
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
  return hip_status(launch_hca_compress(c, z, in_t, B, T, width, ratio, out, out_t, stream),
                    "hca_compress");
}

csa_status csa_compress_append(const void* c_a, const void* c_b, const void* z_a, const void* z_b,
                               csa_dtype in_t, int64_t B, int32_t width, int32_t ratio, const int32_t* pos,
                               void* state, int64_t N_cap, void* out, csa_dtype out_t, void* out_scale,
                               hipStream_t stream) {
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
                                      out_scale, stream),
                    "csa_compress_append");
}

csa_status hca_compress_append(const void* c, const void* z, csa_dtype in_t, int64_t B, int32_t width,
                               int32_t ratio, const int32_t* pos, void* state, int64_t N_cap, void* out,
                               csa_dtype out_t, hipStream_t stream) {
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
                                      stream),
                    "hca_compress_append");
}

size_t indexer_topk_workspace_size(int64_t B, int64_t Tq, int64_t N, int32_t H_I, int32_t d_I, int32_t k,
                                   csa_dtype qk_t) {
  (void)H_I;
  if (B <= 0 || Tq <= 0 || N < 0) return 0;
  return indexer_ws_bytes(B, Tq, N, 4, d_I, qk_t, k);
}

size_t indexer_topk_bf16_scores_workspace_size(int64_t B, int64_t Tq, int64_t N, int32_t H_I, int32_t d_I,
                                               int32_t k, csa_dtype qk_t) {
  (void)H_I;
  if (B <= 0 || Tq <= 0 || N < 0) return 0;
  return indexer_ws_bytes(B, Tq, N, 2, d_I, qk_t, k);
}

static csa_status indexer_common(const char* fn, const void* q_idx, const void* q_scale, const float* w,
                                 const void* k_idx, const void* k_scale, csa_dtype qk_t, const int32_t* q_pos,
                                 int64_t B, int64_t Tq, int64_t N, int32_t H_I, int32_t d_I, int32_t ratio, int32_t k,
                                 int32_t* idx_out, void* score_out, bool bf16, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
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
                                        idx_out, score_out, bf16, ws, stream),
                    fn);
}

csa_status indexer_scores(const void* q_idx, const void* q_scale, const float* w, const void* k_idx,
                          const void* k_scale, csa_dtype qk_t, const int32_t* q_pos, int64_t B, int64_t Tq, int64_t N,
                          int32_t H_I, int32_t d_I, int32_t ratio, float* score_out, hipStream_t stream) {
  g_last_error.clear();
  const char* fn = "indexer_scores";
  CSA_REQUIRE(is_dtype(qk_t), CSA_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, (int)qk_t);
  CSA_REQUIRE(B >= 0 && Tq >= 0 && N >= 0 && N < (int64_t(1) << 30) && B * Tq < (int64_t(1) << 31), CSA_ERR_SHAPE,
              "%s: B=%lld Tq=%lld N=%lld", fn, (long long)B, (long long)Tq, (long long)N);
  CSA_REQUIRE(H_I >= 1 && H_I <= 64, CSA_ERR_UNSUPPORTED, "%s: H_I %d (1..64)", fn, H_I);
  CSA_REQUIRE(d_I == 64 || d_I == 128, CSA_ERR_UNSUPPORTED, "%s: d_I %d (64 or 128)", fn, d_I);
  CSA_REQUIRE(ratio >= 1, CSA_ERR_SHAPE, "%s: ratio %d", fn, ratio);
  const bool quant = qk_t == CSA_FP8_E4M3 || qk_t == CSA_FP4_E2M1;
  CSA_REQUIRE(quant || (q_scale == nullptr && k_scale == nullptr), CSA_ERR_SHAPE,
              "%s: q_scale/k_scale must be NULL for float operands", fn);
  if (B * Tq == 0 || N == 0) return CSA_OK;
  CSA_REQUIRE(q_idx && w && q_pos && k_idx && score_out, CSA_ERR_NULL, "%s: NULL tensor", fn);
  CSA_REQUIRE(!quant || (q_scale && k_scale), CSA_ERR_NULL, "%s: scales required", fn);
  CSA_REQUIRE(((uintptr_t)q_idx & 15) == 0 && ((uintptr_t)k_idx & 15) == 0 && ((uintptr_t)k_scale & 3) == 0,
              CSA_ERR_SHAPE, "%s: q_idx and k_idx must be 16-byte aligned, k_scale 4-byte aligned", fn);
  return hip_status(launch_indexer_scores(q_idx, q_scale, w, k_idx, k_scale, qk_t, q_pos, B, Tq, N, H_I, d_I, ratio,
                                          score_out, stream),
                    fn);
}

csa_status indexer_topk(const void* q_idx, const void* q_scale, const float* w, const void* k_idx,
                        const void* k_scale, csa_dtype qk_t, const int32_t* q_pos, int64_t B, int64_t Tq,
                        int64_t N, int32_t H_I, int32_t d_I, int32_t ratio, int32_t k, int32_t* idx_out,
                        float* score_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  return indexer_common("indexer_topk", q_idx, q_scale, w, k_idx, k_scale, qk_t, q_pos, B, Tq, N, H_I, d_I, ratio,
                        k, idx_out, score_out, false, ws, ws_bytes, stream);
}

csa_status indexer_topk_bf16_scores(const void* q_idx, const void* q_scale, const float* w, const void* k_idx,
                                    const void* k_scale, csa_dtype qk_t, const int32_t* q_pos, int64_t B,
                                    int64_t Tq, int64_t N, int32_t H_I, int32_t d_I, int32_t ratio, int32_t k,
                                    int32_t* idx_out, uint16_t* score_out, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  g_last_error.clear();
  return indexer_common("indexer_topk_bf16_scores", q_idx, q_scale, w, k_idx, k_scale, qk_t, q_pos, B, Tq, N, H_I,
                        d_I, ratio, k, idx_out, score_out, true, ws, ws_bytes, stream);
}

static csa_status check_attn_common(const char* fn, const void* q, const void* kv, const void* x_win,
                                    const int32_t* win_start, const int32_t* q_pos, csa_dtype t, int64_t B,
                                    int64_t Tq, int64_t N, int64_t T_win, int32_t H, int32_t d, int32_t window,
                                    float scale, void* out) {
  CSA_REQUIRE(is_dtype(t), CSA_ERR_UNSUPPORTED, "%s: unknown dtype", fn);
  // the kernels mask keys with a logit of -inf and take the running maximum
  // of unscaled logits: both rely on a positive scale
  CSA_REQUIRE(scale > 0.f && scale <= 3.402823466e38f, CSA_ERR_SHAPE, "%s: scale %g (finite and > 0)", fn,
              (double)scale);
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

static constexpr uint32_t kAttnFlags = CSA_ATTN_WIN_RING | CSA_ATTN_BATCH_INVARIANT;

size_t sparse_attn_workspace_size(int64_t B, int64_t Tq, int32_t H, int32_t d, int32_t k, int32_t window,
                                  uint32_t flags) {
  (void)d;
  if (B <= 0 || Tq <= 0 || H <= 0) return 0;
  return attn_ws_bytes(B, Tq, H, (int64_t)k + window, (flags & CSA_ATTN_BATCH_INVARIANT) != 0);
}

csa_status sparse_attn_fwd(const void* q, const void* kv, const int32_t* idx, const void* x_win,
                           const int32_t* win_start, const float* sink, const int32_t* q_pos, csa_dtype t, int64_t B,
                           int64_t Tq, int64_t N, int64_t T_win, int32_t H, int32_t d, int32_t k, int32_t window,
                           float scale, void* out, float* lse, void* ws, size_t ws_bytes, uint32_t flags,
                           hipStream_t stream) {
  g_last_error.clear();
  csa_status st = check_attn_common("sparse_attn_fwd", q, kv, x_win, win_start, q_pos, t, B, Tq, N, T_win, H, d,
                                    window, scale, out);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(k >= 1 && k <= 4096, CSA_ERR_SHAPE, "sparse_attn_fwd: k %d (1..4096)", k);
  CSA_REQUIRE((flags & ~kAttnFlags) == 0, CSA_ERR_SHAPE, "sparse_attn_fwd: unknown flags 0x%x", flags);
  if (B * Tq == 0) return CSA_OK;
  CSA_REQUIRE(idx, CSA_ERR_NULL, "sparse_attn_fwd: idx is NULL");
  const bool binv = (flags & CSA_ATTN_BATCH_INVARIANT) != 0;
  // one reading of the options: the size checked here is the one the launch plans with
  const size_t need = attn_ws_bytes(B, Tq, H, (int64_t)k + window, binv);
  CSA_REQUIRE(need == 0 || (ws && ws_bytes >= need), CSA_ERR_WORKSPACE, "sparse_attn_fwd: workspace %zu < %zu bytes",
              ws_bytes, need);
  return hip_status(launch_attention(true, t, q, kv, idx, x_win, win_start, sink, q_pos, B, Tq, N, T_win,
                                     (flags & CSA_ATTN_WIN_RING) ? 1 : 0, H, k, window, 1, scale, out, lse,
                                     need ? ws : nullptr, (int64_t)k + window, binv, stream),
                    "sparse_attn_fwd");
}

size_t dense_attn_workspace_size(int64_t B, int64_t Tq, int64_t N, int32_t H, int32_t d, int32_t window,
                                 uint32_t flags) {
  (void)d;
  if (B <= 0 || Tq <= 0 || H <= 0) return 0;
  return attn_ws_bytes(B, Tq, H, N + window, (flags & CSA_ATTN_BATCH_INVARIANT) != 0);
}

csa_status dense_compressed_attn_fwd(const void* q, const void* kv, const void* x_win, const int32_t* win_start,
                                     const float* sink, const int32_t* q_pos, csa_dtype t, int64_t B, int64_t Tq,
                                     int64_t N, int64_t T_win, int32_t H, int32_t d, int32_t ratio, int32_t window,
                                     float scale, void* out, float* lse, void* ws, size_t ws_bytes, uint32_t flags,
                                     hipStream_t stream) {
  g_last_error.clear();
  csa_status st = check_attn_common("dense_compressed_attn_fwd", q, kv, x_win, win_start, q_pos, t, B, Tq, N, T_win,
                                    H, d, window, scale, out);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(ratio >= 1, CSA_ERR_SHAPE, "dense_compressed_attn_fwd: ratio %d", ratio);
  CSA_REQUIRE((flags & ~kAttnFlags) == 0, CSA_ERR_SHAPE, "dense_compressed_attn_fwd: unknown flags 0x%x", flags);
  if (B * Tq == 0) return CSA_OK;
  const bool binv = (flags & CSA_ATTN_BATCH_INVARIANT) != 0;
  const size_t need = attn_ws_bytes(B, Tq, H, N + window, binv);
  CSA_REQUIRE(need == 0 || (ws && ws_bytes >= need), CSA_ERR_WORKSPACE,
              "dense_compressed_attn_fwd: workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(launch_attention(false, t, q, kv, nullptr, x_win, win_start, sink, q_pos, B, Tq, N, T_win,
                                     (flags & CSA_ATTN_WIN_RING) ? 1 : 0, H, 0, window, ratio, scale, out, lse,
                                     need ? ws : nullptr, N + window, binv, stream),
                    "dense_compressed_attn_fwd");
}

// ------------------------------------------------------------------ allocation-free variant
// Scratch for sparse_attn_fwd_noalloc: a file-scope device array that each GPU
// holds from module load until the process ends. Host code never passes the
// array's name to a kernel (on the host it is only a stand-in): the device
// address is looked up once per device with hipGetSymbolAddress.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

static csa_status scratch_address(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, fn);
  CSA_REQUIRE(dev >= 0 && dev < kMaxDevices, CSA_ERR_UNSUPPORTED, "%s: device %d", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, fn);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSA_OK;
}

size_t sparse_attn_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

csa_status sparse_attn_fwd_noalloc(const void* q, const void* kv, const int32_t* idx, const void* x_win,
                                   const int32_t* win_start, const float* sink, const int32_t* q_pos, csa_dtype t,
                                   int64_t B, int64_t Tq, int64_t N, int64_t T_win, int32_t H, int32_t d, int32_t k,
                                   int32_t window, float scale, void* out, float* lse, uint32_t flags,
                                   hipStream_t stream) {
  g_last_error.clear();
  csa_status st = check_attn_common("sparse_attn_fwd_noalloc", q, kv, x_win, win_start, q_pos, t, B, Tq, N, T_win,
                                    H, d, window, scale, out);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(k >= 1 && k <= 4096, CSA_ERR_SHAPE, "sparse_attn_fwd_noalloc: k %d (1..4096)", k);
  CSA_REQUIRE((flags & ~kAttnFlags) == 0, CSA_ERR_SHAPE, "sparse_attn_fwd_noalloc: unknown flags 0x%x", flags);
  if (B * Tq == 0) return CSA_OK;
  CSA_REQUIRE(idx, CSA_ERR_NULL, "sparse_attn_fwd_noalloc: idx is NULL");
  const bool binv = (flags & CSA_ATTN_BATCH_INVARIANT) != 0;
  const size_t need = attn_ws_bytes(B, Tq, H, (int64_t)k + window, binv);
  CSA_REQUIRE(need <= kNoAllocScratchBytes, CSA_ERR_WORKSPACE,
              "sparse_attn_fwd_noalloc: these shapes need %zu bytes of scratch, more than the %zu bytes the "
              "library holds per device (use sparse_attn_fwd with a workspace)",
              need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address("sparse_attn_fwd_noalloc", &ws);
    if (st != CSA_OK) return st;
  }
  return hip_status(launch_attention(true, t, q, kv, idx, x_win, win_start, sink, q_pos, B, Tq, N, T_win,
                                     (flags & CSA_ATTN_WIN_RING) ? 1 : 0, H, k, window, 1, scale, out, lse, ws,
                                     (int64_t)k + window, binv, stream),
                    "sparse_attn_fwd_noalloc");
}

csa_status csa_window_append(const void* x_new, csa_dtype t, int64_t B, int32_t d, const int32_t* pos, void* ring,
                             int64_t R, hipStream_t stream) {
  g_last_error.clear();
  CSA_REQUIRE(is_dtype(t) && is_float(t), CSA_ERR_UNSUPPORTED, "csa_window_append: dtype must be CSA_F32 or CSA_BF16");
  CSA_REQUIRE(d == 128, CSA_ERR_UNSUPPORTED, "csa_window_append: d %d (only 128)", d);
  CSA_REQUIRE(B >= 0 && R >= 1 && B * R < ((int64_t)1 << 40), CSA_ERR_SHAPE, "csa_window_append: B=%lld R=%lld",
              (long long)B, (long long)R);
  if (B == 0) return CSA_OK;
  CSA_REQUIRE(x_new && pos && ring, CSA_ERR_NULL, "csa_window_append: NULL tensor");
  CSA_REQUIRE(((uintptr_t)x_new & 15) == 0 && ((uintptr_t)ring & 15) == 0, CSA_ERR_SHAPE,
              "csa_window_append: x_new and ring must be 16-byte aligned");
  return hip_status(launch_window_append(x_new, t, B, pos, ring, R, stream), "csa_window_append");
}

csa_status csa_state_checkpoint(const void* state, int64_t B, int64_t seq_bytes, const int32_t* pos, int32_t period,
                                void* ckpt, int64_t n_slots, hipStream_t stream) {
  g_last_error.clear();
  const char* fn = "csa_state_checkpoint";
  CSA_REQUIRE(B >= 0 && B <= 65535 && seq_bytes > 0 && seq_bytes % 16 == 0 && period >= 1 && n_slots >= 1,
              CSA_ERR_SHAPE, "%s: B=%lld seq_bytes=%lld period=%d n_slots=%lld", fn, (long long)B,
              (long long)seq_bytes, period, (long long)n_slots);
  if (B == 0) return CSA_OK;
  CSA_REQUIRE(state && pos && ckpt, CSA_ERR_NULL, "%s: NULL tensor", fn);
  CSA_REQUIRE(((uintptr_t)state & 15) == 0 && ((uintptr_t)ckpt & 15) == 0, CSA_ERR_SHAPE,
              "%s: state and ckpt must be 16-byte aligned", fn);
  return hip_status(launch_state_checkpoint(state, B, seq_bytes, pos, period, ckpt, n_slots, stream), fn);
}

csa_status csa_state_restore(const void* ckpt, int64_t B, int64_t seq_bytes, int64_t n_slots, const int32_t* slot,
                             void* state, hipStream_t stream) {
  g_last_error.clear();
  const char* fn = "csa_state_restore";
  CSA_REQUIRE(B >= 0 && B <= 65535 && seq_bytes > 0 && seq_bytes % 16 == 0 && n_slots >= 1, CSA_ERR_SHAPE,
              "%s: B=%lld seq_bytes=%lld n_slots=%lld", fn, (long long)B, (long long)seq_bytes, (long long)n_slots);
  if (B == 0) return CSA_OK;
  CSA_REQUIRE(ckpt && slot && state, CSA_ERR_NULL, "%s: NULL tensor", fn);
  CSA_REQUIRE(((uintptr_t)state & 15) == 0 && ((uintptr_t)ckpt & 15) == 0, CSA_ERR_SHAPE,
              "%s: state and ckpt must be 16-byte aligned", fn);
  return hip_status(launch_state_restore(ckpt, B, seq_bytes, n_slots, slot, state, stream), fn);
}

csa_status csa_ring_fill(const void* hist, int64_t B, int64_t T_hist, int64_t row_bytes, const int32_t* pos,
                         int64_t R, void* ring, hipStream_t stream) {
  g_last_error.clear();
  const char* fn = "csa_ring_fill";
  CSA_REQUIRE(B >= 0 && B <= 65535 && T_hist >= 0 && row_bytes > 0 && row_bytes % 16 == 0 && R >= 1 &&
                  R <= ((int64_t)1 << 31) - 1,
              CSA_ERR_SHAPE, "%s: B=%lld T_hist=%lld row_bytes=%lld R=%lld", fn, (long long)B, (long long)T_hist,
              (long long)row_bytes, (long long)R);
  if (B == 0 || T_hist == 0) return CSA_OK;
  CSA_REQUIRE(hist && pos && ring, CSA_ERR_NULL, "%s: NULL tensor", fn);
  CSA_REQUIRE(((uintptr_t)hist & 15) == 0 && ((uintptr_t)ring & 15) == 0, CSA_ERR_SHAPE,
              "%s: hist and ring must be 16-byte aligned", fn);
  return hip_status(launch_ring_fill(hist, B, T_hist, row_bytes, pos, R, ring, stream), fn);
}

// ------------------------------------------------------------------ projections
static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

csa_status csa_linear_bf16(const void* A, int64_t lda, int64_t sA, const void* W, int64_t ldw, int64_t sW, void* C,
                           csa_dtype out_t, int64_t ldc, int64_t sC, int64_t M, int64_t N, int64_t K, int64_t G,
                           hipStream_t stream) {
  g_last_error.clear();
  const char* fn = "csa_linear_bf16";
  CSA_REQUIRE(out_t == CSA_BF16 || out_t == CSA_F32, CSA_ERR_UNSUPPORTED, "%s: output must be CSA_BF16 or CSA_F32",
              fn);
  CSA_REQUIRE(M >= 0 && N >= 0 && K >= 0 && G >= 0 && M < ((int64_t)1 << 31) && N < ((int64_t)1 << 31) && G <= 65535,
              CSA_ERR_SHAPE, "%s: M=%lld N=%lld K=%lld G=%lld", fn, (long long)M, (long long)N, (long long)K,
              (long long)G);
  CSA_REQUIRE(K % 64 == 0, CSA_ERR_SHAPE, "%s: K=%lld must be a multiple of 64", fn, (long long)K);
  if (M * N * G == 0) return CSA_OK;
  // one block per 128 x 128 tile of C: the launch's work-item count must fit 32 bits
  CSA_REQUIRE(((M + 127) / 128) * ((N + 127) / 128) < ((int64_t)1 << 24), CSA_ERR_SHAPE,
              "%s: M=%lld x N=%lld has too many 128 x 128 tiles for one launch (at most 2^24 - 1)", fn,
              (long long)M, (long long)N);
  CSA_REQUIRE(K > 0, CSA_ERR_SHAPE, "%s: K must be positive", fn);
  CSA_REQUIRE(A && W && C, CSA_ERR_NULL, "%s: NULL tensor", fn);
  CSA_REQUIRE(lda >= K && ldw >= K && ldc >= N, CSA_ERR_SHAPE, "%s: lda=%lld ldw=%lld ldc=%lld", fn, (long long)lda,
              (long long)ldw, (long long)ldc);
  CSA_REQUIRE(lda % 8 == 0 && ldw % 8 == 0 && sA % 8 == 0 && sW % 8 == 0 && aligned16(A) && aligned16(W) &&
                  ((uintptr_t)C & (out_t == CSA_BF16 ? 1 : 3)) == 0,
              CSA_ERR_SHAPE, "%s: A and W need 16-byte aligned rows (base 16-byte aligned, strides multiples of 8 "
              "elements); C must be aligned to its element size", fn);
  return hip_status(launch_gemm_bf16(A, lda, sA, W, ldw, sW, C, ldc, sC, M, N, K, G, out_t == CSA_BF16, stream), fn);
}

size_t csa_grouped_out_proj_workspace_size(int64_t T, int32_t G, int32_t r) {
  if (T <= 0 || G <= 0 || r <= 0) return 0;
  return ((size_t)T * G * r * 2 + 255) / 256 * 256;
}

csa_status csa_grouped_out_proj(const void* o, const void* w_group, const void* w_out, int64_t T, int32_t H, int32_t d,
                                int32_t G, int32_t r, int32_t D, void* out, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  g_last_error.clear();
  const char* fn = "csa_grouped_out_proj";
  CSA_REQUIRE(T >= 0 && H >= 1 && d >= 1 && G >= 1 && r >= 1 && D >= 1 && H % G == 0, CSA_ERR_SHAPE,
              "%s: T=%lld H=%d d=%d G=%d r=%d D=%d (G must divide H)", fn, (long long)T, H, d, G, r, D);
  const int64_t Kg = (int64_t)(H / G) * d;
  CSA_REQUIRE(Kg % 64 == 0 && ((int64_t)G * r) % 64 == 0, CSA_ERR_SHAPE,
              "%s: (H/G)*d and G*r must be multiples of 64", fn);
  if (T == 0) return CSA_OK;
  CSA_REQUIRE(o && w_group && w_out && out, CSA_ERR_NULL, "%s: NULL tensor", fn);
  const size_t need = csa_grouped_out_proj_workspace_size(T, G, r);
  CSA_REQUIRE(ws && ws_bytes >= need, CSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  // y[:, g*r : (g+1)*r] = o[:, g*Kg : (g+1)*Kg] * w_group[g]^T   (bf16 group results)
  csa_status st = csa_linear_bf16(o, (int64_t)H * d, Kg, w_group, Kg, (int64_t)r * Kg, ws, CSA_BF16, (int64_t)G * r,
                                  r, T, r, Kg, G, stream);
  if (st != CSA_OK) return st;
  // out = y * w_out^T
  return csa_linear_bf16(ws, (int64_t)G * r, 0, w_out, (int64_t)G * r, 0, out, CSA_BF16, D, 0, T, D, (int64_t)G * r,
                         1, stream);
}

size_t csa_query_proj_shared_workspace_size(int64_t T, int32_t r_q) {
  if (T <= 0 || r_q <= 0) return 0;
  return ((size_t)T * r_q * 2 + 255) / 256 * 256;
}

csa_status csa_query_proj_shared(const void* x, const void* w_dq, const void* w_uq, const void* w_iq, int64_t T,
                                 int32_t D, int32_t r_q, int32_t n_q, int32_t n_i, void* q, void* q_idx, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  const char* fn = "csa_query_proj_shared";
  CSA_REQUIRE(T >= 0 && D >= 1 && r_q >= 1 && n_q >= 1 && n_i >= 1, CSA_ERR_SHAPE,
              "%s: T=%lld D=%d r_q=%d n_q=%d n_i=%d", fn, (long long)T, D, r_q, n_q, n_i);
  CSA_REQUIRE(D % 64 == 0 && r_q % 64 == 0, CSA_ERR_SHAPE, "%s: D and r_q must be multiples of 64", fn);
  if (T == 0) return CSA_OK;
  CSA_REQUIRE(x && w_dq && w_uq && w_iq && q && q_idx, CSA_ERR_NULL, "%s: NULL tensor", fn);
  const size_t need = csa_query_proj_shared_workspace_size(T, r_q);
  CSA_REQUIRE(ws && ws_bytes >= need, CSA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  csa_status st = csa_linear_bf16(x, D, 0, w_dq, D, 0, ws, CSA_BF16, r_q, 0, T, r_q, D, 1, stream);   // shared latent
  if (st != CSA_OK) return st;
  st = csa_linear_bf16(ws, r_q, 0, w_uq, r_q, 0, q, CSA_BF16, n_q, 0, T, n_q, r_q, 1, stream);       // attention queries
  if (st != CSA_OK) return st;
  return csa_linear_bf16(ws, r_q, 0, w_iq, r_q, 0, q_idx, CSA_BF16, n_i, 0, T, n_i, r_q, 1, stream); // indexer queries
}

csa_status csa_kv_proj(const void* x, const void* w, int64_t T, int32_t D, int32_t n_streams, int32_t width,
                       void* streams, csa_dtype out_t, hipStream_t stream) {
  g_last_error.clear();
  const char* fn = "csa_kv_proj";
  CSA_REQUIRE(out_t == CSA_BF16 || out_t == CSA_F32, CSA_ERR_UNSUPPORTED, "%s: output must be CSA_BF16 or CSA_F32",
              fn);
  CSA_REQUIRE(T >= 0 && D >= 1 && n_streams >= 1 && n_streams <= 65535 && width >= 1, CSA_ERR_SHAPE,
              "%s: T=%lld D=%d n_streams=%d width=%d", fn, (long long)T, D, n_streams, width);
  CSA_REQUIRE(D % 64 == 0, CSA_ERR_SHAPE, "%s: D=%d must be a multiple of 64", fn, D);
  if (T == 0) return CSA_OK;
  CSA_REQUIRE(x && w && streams, CSA_ERR_NULL, "%s: NULL tensor", fn);
  // stream s = x * w[s]^T: one group per stream, every group reading the same x
  return csa_linear_bf16(x, D, 0, w, D, (int64_t)width * D, streams, out_t, width, T * width, T, width, D,
                         n_streams, stream);
}

static csa_status check_attn_bwd(const char* fn, const void* q, const void* kv, const void* x_win,
                                 const int32_t* win_start, const float* sink, const int32_t* q_pos, csa_dtype t,
                                 int64_t B, int64_t Tq, int64_t N, int64_t T_win, int32_t H, int32_t d,
                                 int32_t window, float scale, const void* out, const float* lse, const void* dout,
                                 void* dq, float* dkv, float* dx_win, float* dsink) {
  csa_status st = check_attn_common(fn, q, kv, x_win, win_start, q_pos, t, B, Tq, N, T_win, H, d, window, scale,
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
                           float* dx_win, float* dsink, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  csa_status st = check_attn_bwd("sparse_attn_bwd", q, kv, x_win, win_start, sink, q_pos, t, B, Tq, N, T_win, H, d,
                                 window, scale, out, lse, dout, dq, dkv, dx_win, dsink);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(k >= 1 && k <= 4096, CSA_ERR_SHAPE, "sparse_attn_bwd: k %d (1..4096)", k);
  if (B * Tq == 0) return CSA_OK;
  CSA_REQUIRE(idx, CSA_ERR_NULL, "sparse_attn_bwd: idx is NULL");
  const size_t need = sparse_attn_bwd_workspace_size(B, Tq, N, T_win, H, d, k, window);
  CSA_REQUIRE(ws && ws_bytes >= need, CSA_ERR_WORKSPACE, "sparse_attn_bwd: workspace %zu < %zu bytes", ws_bytes,
              need);
  return hip_status(launch_attn_bwd(true, q, kv, idx, x_win, win_start, sink, q_pos, out, lse, dout, B, Tq, N, T_win,
                                    H, k, window, 1, scale, dq, dkv, dx_win, dsink, ws, stream),
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
                                     hipStream_t stream) {
  g_last_error.clear();
  csa_status st = check_attn_bwd("dense_compressed_attn_bwd", q, kv, x_win, win_start, sink, q_pos, t, B, Tq, N,
                                 T_win, H, d, window, scale, out, lse, dout, dq, dkv, dx_win, dsink);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(ratio >= 1, CSA_ERR_SHAPE, "dense_compressed_attn_bwd: ratio %d", ratio);
  if (B * Tq == 0) return CSA_OK;
  const size_t need = dense_attn_bwd_workspace_size(B, Tq, N, T_win, H, d, window);
  CSA_REQUIRE(ws && ws_bytes >= need, CSA_ERR_WORKSPACE, "dense_compressed_attn_bwd: workspace %zu < %zu bytes",
              ws_bytes, need);
  return hip_status(launch_attn_bwd(false, q, kv, nullptr, x_win, win_start, sink, q_pos, out, lse, dout, B, Tq, N,
                                    T_win, H, 0, window, ratio, scale, dq, dkv, dx_win, dsink, ws,
                                    stream),
                    "dense_compressed_attn_bwd");
}

csa_status csa_kernel_timer_start(int32_t kernel_id, int32_t max_launches) {
  g_last_error.clear();
  CSA_REQUIRE(kernel_id >= CSA_KID_COMPRESS && kernel_id <= CSA_KID_GEMM, CSA_ERR_SHAPE,
              "csa_kernel_timer_start: kernel id %d", kernel_id);
  CSA_REQUIRE(max_launches >= 1 && max_launches <= kMaxTimed, CSA_ERR_SHAPE,
              "csa_kernel_timer_start: max_launches %d (1..%d)", max_launches, kMaxTimed);
  std::lock_guard<std::mutex> lock(g_timer.mu);
  if (!g_timer.created) {
    for (int i = 0; i < 2 * kMaxTimed; ++i) {
      hipError_t e = hipEventCreate(&g_timer.ev[i]);
      if (e != hipSuccess) return hip_status(e, "csa_kernel_timer_start");
    }
    g_timer.created = true;
  }
  g_timer.cap = max_launches;
  g_timer.n = 0;
  g_timer.kid.store(kernel_id);
  return CSA_OK;
}

int32_t csa_kernel_timer_read(float* ms_out, int32_t capacity) {
  std::lock_guard<std::mutex> lock(g_timer.mu);
  const int n = g_timer.n;
  g_timer.kid.store(0);
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
