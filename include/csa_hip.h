/*
 * csa_hip.h — C ABI of the CSA/HCA hybrid attention forward for MI355X (gfx950).
 *
 * The method is DeepSeek-V4's attention layer as the public write-ups describe
 * it: a gated, overlapped 4:1 KV compressor feeding a low-precision lightning
 * indexer that picks the top-k compressed entries per query (CSA), a 128:1
 * compressor with dense attention over all entries (HCA), and in both a
 * 128-token uncompressed sliding window and a learnable attention sink.
 * Sources, by page address and section:
 *   cf-1.com write-up (www.cf-1.com/news/5231315): §2.4 top-k 512/1024,
 *     §3.1 CSA, §3.2 HCA, §3.3 window branch and sink, §3.4 low-rank FP4
 *     indexer, §4.3 deterministic kernels, §4.4 FP4 QK path, FP4->FP8 lossless.
 *   yfxerp.com write-up "DeepSeek-V4 原理拆解" (www.yfxerp.com/news/211352):
 *     §1 module overview, §3 config skeleton (kv_compress_ratio 4,
 *     top_k_blocks 1024, indexer_rank 64, sliding_window 128,
 *     compress_ratio 128, attention_sink).
 *
 * Conventions (all entry points):
 *  - Every tensor pointer is a DEVICE pointer, allocated, owned and freed by
 *    the caller. Tensors are dense, row-major, with the shapes given below.
 *  - The library never allocates device memory in these calls. Scratch space
 *    is the caller's `ws` buffer, sized by the matching *_workspace_size().
 *  - `stream` is the hipStream_t to enqueue on (NULL = the default stream).
 *    Work is enqueued asynchronously; the caller synchronises before reading
 *    results. C callers compile with -D__HIP_PLATFORM_AMD__ (the HIP runtime
 *    header that defines hipStream_t requires it).
 *  - Arguments are validated on the host before anything is launched. On
 *    failure the call returns a non-zero csa_status, launches nothing, and
 *    csa_last_error() holds a description (thread-local). A failed kernel
 *    launch returns CSA_ERR_HIP. There are no slow fallbacks: an unsupported
 *    combination returns CSA_ERR_UNSUPPORTED.
 *  - Positions are absolute token positions. q_pos unifies prefill (0..T-1),
 *    decode (one position L per sequence) and chunked prefill (L-C..L-1).
 *  - Entry visibility is causal: with compression ratio m, the query at
 *    position p sees entries j < n(p) = min(N, floor((p+1)/m)).
 *  - Results are deterministic: the same inputs give bit-identical outputs.
 *    Results and workspace sizes depend only on the arguments: the library
 *    keeps no mode state between calls.
 */
#ifndef CSA_HIP_H
#define CSA_HIP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_OK = 0,
  CSA_ERR_NULL = 1,        /* a required pointer is NULL */
  CSA_ERR_SHAPE = 2,       /* sizes are negative, inconsistent or out of range */
  CSA_ERR_UNSUPPORTED = 3, /* valid but not implemented (dtype, width, head count) */
  CSA_ERR_WORKSPACE = 4,   /* ws is NULL or smaller than *_workspace_size() */
  CSA_ERR_HIP = 5          /* the HIP runtime reported an error */
} csa_status;

typedef enum {
  CSA_F32 = 0,       /* IEEE float32 */
  CSA_BF16 = 1,      /* bfloat16 (stored as 16-bit words) */
  CSA_FP8_E4M3 = 2,  /* OCP e4m3 (max 448), one float32 scale per row */
  CSA_FP4_E2M1 = 3   /* OCP e2m1, two per byte (element 2i in the low nibble),
                        one E8M0 scale byte per 32 consecutive elements */
} csa_dtype;

/* Human-readable name of a status code (static string). */
const char* csa_status_string(int status);
/* Detail of the last failure on the calling thread ("" if none). */
const char* csa_last_error(void);
/* Library version string. */
const char* csa_version(void);

/*
 * csa_quantize_rows — quantise `rows` vectors of `width` elements.
 * Low-precision indexer keys and queries (cf-1.com write-up §3.4: the indexer
 * QK runs in FP4; §4.4: FP4->FP8 dequantisation is lossless).
 *   x        [rows, width] of in_t (CSA_F32 or CSA_BF16)
 *   out      CSA_FP8_E4M3: uint8 [rows, width]; scale: float32 [rows],
 *              scale = amax/448 in float32 (1 for an all-zero row),
 *              code = e4m3(x / scale), IEEE float32 division, round to
 *              nearest even, saturating at 448.
 *            CSA_FP4_E2M1: uint8 [rows, width/2]; scale: uint8 [rows, width/32]
 *              holding E+127 with E = floor(log2(block amax)) - 2 (0 for an
 *              all-zero block), code = e2m1(x * 2^-E), round to nearest even,
 *              saturating at 6.
 *   width    multiple of 32 (fp4) or any positive value (fp8), <= 4096.
 * The sign bit of a code is the sign of the input (tiny negatives give -0).
 */
csa_status csa_quantize_rows(const void* x, csa_dtype in_t, int64_t rows, int32_t width,
                             void* out, csa_dtype out_t, void* scale, hipStream_t stream);

/*
 * csa_compress — CSA compressor: overlapped, gated, two-stream, ratio:1
 * (cf-1.com write-up §3.1; yfxerp.com write-up §3 kv_compress_ratio 4).
 * Entry j, channel c:  E[j,c] = sum_t w_t * C_t[c], with one softmax per
 * channel over the joint list of gate logits of stream A at tokens
 * [ratio*j, ratio*j+ratio) and stream B at tokens [ratio*j-ratio, ratio*j)
 * (B omitted for j = 0). N = floor(T/ratio); a trailing partial block is
 * not compressed.
 *   c_a, c_b, z_a, z_b  [B, T, width] of in_t (CSA_F32 or CSA_BF16)
 *   out       [B, N, width] of out_t: CSA_F32, CSA_BF16, or a quantised
 *             indexer-key format (CSA_FP8_E4M3 / CSA_FP4_E2M1, quantised per
 *             entry row exactly as csa_quantize_rows does, from the float32
 *             value of E) with out_scale as csa_quantize_rows' `scale`
 *             ([B, N] float32 or [B, N, width/32] uint8). out_scale must be
 *             NULL for CSA_F32/CSA_BF16.
 *   width     64 or 128;  ratio 1..128.
 */
csa_status csa_compress(const void* c_a, const void* c_b, const void* z_a, const void* z_b,
                        csa_dtype in_t, int64_t B, int64_t T, int32_t width, int32_t ratio,
                        void* out, csa_dtype out_t, void* out_scale, hipStream_t stream);

/*
 * hca_compress — HCA compressor: non-overlapped, gated, single stream,
 * ratio:1 (cf-1.com write-up §3.2; yfxerp.com write-up §3 compress_ratio 128).
 * E[j,c] = sum_{i<ratio} softmax_i(Z[ratio*j+i, c]) * C[ratio*j+i, c].
 * Ratio 1 is the identity.
 *   c, z   [B, T, width] of in_t (CSA_F32 or CSA_BF16)
 *   out    [B, floor(T/ratio), width] of out_t (CSA_F32 or CSA_BF16)
 *   width  64 or 128;  ratio 1..4096.
 */
csa_status hca_compress(const void* c, const void* z, csa_dtype in_t, int64_t B, int64_t T,
                        int32_t width, int32_t ratio, void* out, csa_dtype out_t, hipStream_t stream);

/*
 * csa_compress_append — decode-time step of the CSA compressor (cf-1.com
 * write-up §4.4: the KV cache keeps a state cache of recent uncompressed
 * tokens beside the compressed entries; §3.1: entry j is made from stream A
 * of block j and stream B of block j-1). For each sequence b, the new token's
 * rows at absolute position pos[b] go into the sequence's state ring; when
 * the token completes block j = (pos[b]+1)/ratio - 1 (and j < N_cap), entry
 * j is computed exactly as csa_compress computes it (same device code: the
 * same bits) and written to row j of the sequence's cache.
 *   c_a, c_b, z_a, z_b  [B, width] of in_t: the new token of each sequence
 *   pos       int32 [B]: its position; a negative position skips the sequence
 *   state     [B, 2*ratio, 4, width] of in_t, caller-owned and persistent:
 *             tokens t of the last 2*ratio positions at slot t % (2*ratio),
 *             streams in the order c_a, c_b, z_a, z_b. Before the first
 *             append of a sequence starting at position p0 > 0, slots of the
 *             2*ratio - 1 tokens before p0 must hold those tokens (appending
 *             them, with their outputs discarded, does it).
 *   out       [B, N_cap, width] of out_t (and out_scale as in csa_compress:
 *             [B, N_cap] float32 for fp8, [B, N_cap, width/32] uint8 for fp4)
 *   width 64 or 128; ratio 1..128. Sequences of one call must be distinct.
 */
csa_status csa_compress_append(const void* c_a, const void* c_b, const void* z_a, const void* z_b,
                               csa_dtype in_t, int64_t B, int32_t width, int32_t ratio, const int32_t* pos,
                               void* state, int64_t N_cap, void* out, csa_dtype out_t, void* out_scale,
                               hipStream_t stream);

/*
 * hca_compress_append — decode-time step of the HCA compressor (cf-1.com
 * write-up §4.4 state cache; §3.2: one entry per 128 tokens). The new token
 * (rows of c and z) at position pos[b] goes into the sequence's ring of the
 * last ratio tokens; when it completes block j = (pos[b]+1)/ratio - 1 (and
 * j < N_cap), entry j is computed exactly as hca_compress computes it and
 * written to row j of the sequence's cache.
 *   c, z   [B, width] of in_t (CSA_F32 or CSA_BF16)
 *   pos    int32 [B]; a negative position skips the sequence
 *   state  [B, ratio, 2, width] of in_t, caller-owned and persistent: token t
 *          at slot t % ratio, streams c, z. Block j's first ratio - 1 tokens
 *          must have been appended (or written there) before its last one.
 *   out    [B, N_cap, width] of out_t (CSA_F32 or CSA_BF16)
 *   width 64 or 128; ratio 1..4096.
 */
csa_status hca_compress_append(const void* c, const void* z, csa_dtype in_t, int64_t B, int32_t width,
                               int32_t ratio, const int32_t* pos, void* state, int64_t N_cap, void* out,
                               csa_dtype out_t, hipStream_t stream);

/*
 * indexer_topk — lightning-indexer scores and per-query top-k selection
 * (cf-1.com write-up §3.1: each query picks its top-k compressed entries
 * through the lightning indexer; §2.4: k = 512 or 1024; §3.4: low-rank,
 * low-precision indexer; yfxerp.com write-up §3 top_k_blocks, indexer_rank).
 * Score of entry s for the query at position p (s < n(p)):
 *     I(p,s) = sum_h w(p,h) * max(0, q(p,h) . k(s))
 * with q and k dequantised (code * scale). Scores are accumulated in float32.
 * Selection: the min(k, n(p)) largest scores under the total order
 * (score descending, index ascending); -0 equals +0.
 *   q_idx    [B, Tq, H_I, d_I] of qk_t (fp4: [B, Tq, H_I, d_I/2] bytes)
 *   q_scale  fp8: float32 [B, Tq, H_I]; fp4: uint8 [B, Tq, H_I, d_I/32];
 *            must be NULL for CSA_F32 / CSA_BF16
 *   w        float32 [B, Tq, H_I], any sign
 *   k_idx    [B, N, d_I] of qk_t;  k_scale: fp8 float32 [B, N], fp4 uint8
 *            [B, N, d_I/32], NULL otherwise
 *   q_pos    int32 [B, Tq], >= 0
 *   idx_out  int32 [B, Tq, k]: selected entries in ascending order, then -1
 *   score_out  NULL, or float32 [B, Tq, N]: the scores (entries >= n(p)
 *            are left untouched)
 *   H_I 1..64; d_I 64 or 128; k 1..2048; ratio >= 1; N < 2^30; B*Tq < 2^31.
 *   q_idx and k_idx must be 16-byte aligned, k_scale 4-byte aligned
 *   (CSA_ERR_SHAPE otherwise).
 * Scores must be finite (NaN selection order is undefined).
 */
size_t indexer_topk_workspace_size(int64_t B, int64_t Tq, int64_t N, int32_t H_I, int32_t d_I,
                                   int32_t k, csa_dtype qk_t);
csa_status indexer_topk(const void* q_idx, const void* q_scale, const float* w,
                        const void* k_idx, const void* k_scale, csa_dtype qk_t,
                        const int32_t* q_pos, int64_t B, int64_t Tq, int64_t N,
                        int32_t H_I, int32_t d_I, int32_t ratio, int32_t k,
                        int32_t* idx_out, float* score_out, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/*
 * indexer_scores — the score stage of indexer_topk on its own (cf-1.com
 * write-up §3.1, §3.4): I(p,s) for every visible entry s < n(p), exactly as
 * indexer_topk computes them (same kernels, same bits), written to
 * score_out float32 [B, Tq, N] (entries >= n(p) untouched); no selection and
 * no workspace. Arguments, layouts, limits and errors are those of
 * indexer_topk without k, idx_out and the workspace.
 */
csa_status indexer_scores(const void* q_idx, const void* q_scale, const float* w, const void* k_idx,
                          const void* k_scale, csa_dtype qk_t, const int32_t* q_pos, int64_t B, int64_t Tq,
                          int64_t N, int32_t H_I, int32_t d_I, int32_t ratio, float* score_out,
                          hipStream_t stream);

/*
 * indexer_topk_bf16_scores — indexer_topk with bfloat16 index scores
 * (cf-1.com write-up §4.4: quantising the index scores from FP32 to BF16
 * halves the selector's score traffic at a small recall cost).
 * Each score I(p,s) is accumulated in float32 exactly as in indexer_topk,
 * then rounded once to bfloat16 (round to nearest, ties to even); the
 * selection runs on the rounded values under the same total order (score
 * descending, index ascending; -0 equals +0), so entries whose float32
 * scores differ but round to the same bfloat16 value tie and the lower
 * index wins. Arguments, layouts, limits and errors are those of
 * indexer_topk, except:
 *   score_out  NULL, or bfloat16 bits uint16 [B, Tq, N]: the rounded scores
 *              (entries >= n(p) are left untouched)
 *   the workspace is the one indexer_topk_bf16_scores_workspace_size
 *   returns (smaller than indexer_topk's for long rows).
 */
size_t indexer_topk_bf16_scores_workspace_size(int64_t B, int64_t Tq, int64_t N, int32_t H_I,
                                               int32_t d_I, int32_t k, csa_dtype qk_t);
csa_status indexer_topk_bf16_scores(const void* q_idx, const void* q_scale, const float* w,
                                    const void* k_idx, const void* k_scale, csa_dtype qk_t,
                                    const int32_t* q_pos, int64_t B, int64_t Tq, int64_t N,
                                    int32_t H_I, int32_t d_I, int32_t ratio, int32_t k,
                                    int32_t* idx_out, uint16_t* score_out, void* ws,
                                    size_t ws_bytes, hipStream_t stream);

/*
 * Options of the two attention calls and their workspace queries, OR-ed into
 * `flags` (0 = none; other bits are rejected with CSA_ERR_SHAPE):
 *  CSA_ATTN_WIN_RING         x_win is a ring of T_win rows (cf-1.com write-up
 *                            §4.4: the window of recent uncompressed tokens is
 *                            kept as a state cache) and position t is row
 *                            t mod T_win, for the positions win_start ..
 *                            win_start + T_win - 1 (csa_window_append keeps
 *                            it). Without it position t is row t - win_start.
 *  CSA_ATTN_BATCH_INVARIANT  batch-invariant planning (cf-1.com write-up §4.3:
 *                            the kernel library is batch-invariant and
 *                            deterministic): key splits and tile streams are
 *                            planned from one sequence's query count Tq
 *                            instead of the batch's B*Tq, so each sequence's
 *                            output and LSE are the same bits whatever else
 *                            is in the batch. The workspace query must be
 *                            given the same flag as the call it sizes.
 * Every result is deterministic with and without these options.
 */
enum { CSA_ATTN_WIN_RING = 1, CSA_ATTN_BATCH_INVARIANT = 2 };

/*
 * sparse_attn_fwd — CSA core attention over the selected compressed entries,
 * the uncompressed window and the sink (cf-1.com write-up §3.1, §3.3;
 * yfxerp.com write-up §3 sliding_window 128, attention_sink).
 * For the query at position p and head h, with keys (= values, one shared KV
 * head for all query heads) K = {kv[s] : s in idx[p], 0 <= s < N} joined with
 * the window rows of positions max(0, p-window+1) <= t <= p that x_win holds
 * (win_start <= t < win_start + T_win):
 *     l_i = scale * q_h . K_i,
 *     o_h = sum_i e^{l_i} K_i / (e^{sink_h} + sum_i e^{l_i}),
 *     lse_h = log(e^{sink_h} + sum_i e^{l_i}).
 * Entries of idx outside [0, N) (e.g. -1 padding) are skipped.
 *   q      [B, Tq, H, d] of t (CSA_F32 or CSA_BF16)
 *   kv     [B, N, d] of t;   idx int32 [B, Tq, k]
 *   x_win  [B, T_win, d] of t;  win_start int32 [B]: the first position the
 *          rows hold (row layout: see CSA_ATTN_WIN_RING)
 *   sink   float32 [H], or NULL for no sink
 *   q_pos  int32 [B, Tq];  out [B, Tq, H, d] of t;  lse NULL or float32 [B, Tq, H]
 *   ws     the workspace sparse_attn_workspace_size() returns for the same
 *          shapes and flags (NULL allowed when it returns 0)
 *   flags  CSA_ATTN_* options
 *   scale  the softmax scale (e.g. 1/sqrt(d)): finite and > 0, else CSA_ERR_SHAPE
 *   d == 128; H a multiple of 16, <= 256; 1 <= k <= 4096; window >= 0; B*Tq < 2^31.
 * Accumulation is float32; a query with no keys and no sink gives o = 0 and
 * lse = -inf.
 */
size_t sparse_attn_workspace_size(int64_t B, int64_t Tq, int32_t H, int32_t d, int32_t k,
                                  int32_t window, uint32_t flags);
csa_status sparse_attn_fwd(const void* q, const void* kv, const int32_t* idx, const void* x_win,
                           const int32_t* win_start, const float* sink, const int32_t* q_pos,
                           csa_dtype t, int64_t B, int64_t Tq, int64_t N, int64_t T_win,
                           int32_t H, int32_t d, int32_t k, int32_t window, float scale,
                           void* out, float* lse, void* ws, size_t ws_bytes, uint32_t flags,
                           hipStream_t stream);

/*
 * sparse_attn_fwd_noalloc — sparse_attn_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, formula, layouts, flags, limits and
 * results as sparse_attn_fwd, without ws / ws_bytes: the split partial results
 * go to a scratch array of sparse_attn_noalloc_scratch_bytes() bytes (32 MiB)
 * that the library holds on each GPU it runs on, from the library's load until
 * the process ends. Shapes whose sparse_attn_workspace_size() exceeds it are
 * rejected with CSA_ERR_WORKSPACE before anything is launched. The call makes
 * no allocation (no hipMalloc, hipFree or allocating library routine). Every
 * call on one GPU shares that GPU's scratch: calls that overlap on one GPU
 * (other streams, other threads) race and must be ordered by the caller.
 */
size_t sparse_attn_noalloc_scratch_bytes(void);
csa_status sparse_attn_fwd_noalloc(const void* q, const void* kv, const int32_t* idx, const void* x_win,
                                   const int32_t* win_start, const float* sink, const int32_t* q_pos,
                                   csa_dtype t, int64_t B, int64_t Tq, int64_t N, int64_t T_win,
                                   int32_t H, int32_t d, int32_t k, int32_t window, float scale,
                                   void* out, float* lse, uint32_t flags, hipStream_t stream);

/*
 * dense_compressed_attn_fwd — HCA core attention: every visible compressed
 * entry (j < n(p), dense, no selection), plus the window and the sink
 * (cf-1.com write-up §3.2, §3.3). Same formula, layouts, flags and limits as
 * sparse_attn_fwd with idx = 0..n(p)-1.
 *   ratio >= 1 defines n(p); B*Tq < 2^31.
 */
size_t dense_attn_workspace_size(int64_t B, int64_t Tq, int64_t N, int32_t H, int32_t d,
                                 int32_t window, uint32_t flags);
csa_status dense_compressed_attn_fwd(const void* q, const void* kv, const void* x_win,
                                     const int32_t* win_start, const float* sink,
                                     const int32_t* q_pos, csa_dtype t, int64_t B, int64_t Tq,
                                     int64_t N, int64_t T_win, int32_t H, int32_t d,
                                     int32_t ratio, int32_t window, float scale, void* out,
                                     float* lse, void* ws, size_t ws_bytes, uint32_t flags,
                                     hipStream_t stream);

/*
 * csa_window_append — one decode step of the window state cache (cf-1.com
 * write-up §4.4: recent uncompressed tokens are kept in a state cache; §3.3:
 * their KV forms the window branch): ring[b, pos[b] mod R] = x_new[b].
 *   x_new  [B, d] of t (CSA_F32 or CSA_BF16): the new token's window row
 *          (the raw KV vector that the attention reads as a window key)
 *   pos    int32 [B]: the token's position; a negative position skips the sequence
 *   ring   [B, R, d] of t, caller-owned, R >= 1
 * d == 128; x_new and ring 16-byte aligned. After appending position p with
 * R >= window, pass x_win = ring, T_win = R, the CSA_ATTN_WIN_RING flag and
 * win_start = max(0, p - R + 1) to the attention calls.
 */
csa_status csa_window_append(const void* x_new, csa_dtype t, int64_t B, int32_t d,
                             const int32_t* pos, void* ring, int64_t R, hipStream_t stream);

/*
 * State cache for resuming at a prefix (cf-1.com write-up §4.4: the KV cache
 * is split into a state cache and a classical KV cache, with three trade-offs
 * for the recent uncompressed tokens: full SWA caching, periodic
 * checkpointing every 1024 tokens, zero SWA caching). A sequence's state
 * cache is its decode-time rings: the window ring [B, R, d]
 * (csa_window_append), the CSA compressor ring [B, 2*ratio, 4, width] and the
 * HCA compressor ring [B, ratio, 2, width] (csa_compress_append,
 * hca_compress_append); the compressed entries are the classical cache. Each
 * call below treats one ring tensor, seq_bytes (or row_bytes) per sequence,
 * as bytes: a multiple of 16, 16-byte aligned; B <= 65535.
 *
 * csa_state_checkpoint — periodic checkpointing. After the token at position
 * pos[b] has been appended, a sequence with pos[b] >= 0 and
 * (pos[b] + 1) % period == 0 copies its ring, state[b] (seq_bytes), to
 * ckpt[b, (pos[b] + 1) / period - 1] (skipped past n_slots); other sequences
 * are untouched. ckpt: [B, n_slots, seq_bytes] bytes, caller-owned.
 */
csa_status csa_state_checkpoint(const void* state, int64_t B, int64_t seq_bytes, const int32_t* pos,
                                int32_t period, void* ckpt, int64_t n_slots, hipStream_t stream);

/*
 * csa_state_restore — state[b] = ckpt[b, slot[b]] for 0 <= slot[b] < n_slots
 * (other sequences untouched). To resume at position P from checkpoint
 * c = P / period - 1 (>= 0), restore slot c and append tokens
 * period * (c + 1) .. P - 1 again: the rings then hold exactly what an
 * uninterrupted run holds after appending position P - 1.
 */
csa_status csa_state_restore(const void* ckpt, int64_t B, int64_t seq_bytes, int64_t n_slots,
                             const int32_t* slot, void* state, hipStream_t stream);

/*
 * csa_ring_fill — full SWA caching: a ring rebuilt from a full-length
 * history of its rows. hist [B, T_hist, row_bytes] holds the row of every
 * position (the window row, or a compressor ring slot's stream rows
 * interleaved as in the ring); ring [B, R, row_bytes]. For each sequence,
 * ring[b, t % R] = hist[b, t] for max(0, pos[b] - R) <= t < pos[b] and
 * t < T_hist (other rows untouched): the ring as an uninterrupted run leaves
 * it after appending position pos[b] - 1. Zero SWA caching needs no call:
 * appending the last max(R) positions again rebuilds every ring.
 */
csa_status csa_ring_fill(const void* hist, int64_t B, int64_t T_hist, int64_t row_bytes,
                         const int32_t* pos, int64_t R, void* ring, hipStream_t stream);

/*
 * Projections around the attention core (cf-1.com write-up §3.4: the
 * lightning indexer shares projection parameters with the main attention;
 * the grouped output projection splits the many query heads (128 in V4-Pro)
 * into groups, reduces each group's dimension, concatenates the groups and
 * projects, cutting the output projection's parameters and FLOPs). The pages
 * give no group count, rank or model width: all are arguments.
 *
 * csa_linear_bf16 — C[g] = A[g] * W[g]^T for g < G: A[g] [M, K] (row stride
 * lda), W[g] [N, K] (a linear layer's [out, in] weight, row stride ldw),
 * C[g] [M, N] (row stride ldc) of out_t (CSA_BF16, rounded to nearest even,
 * or CSA_F32); group g's A, W and C start sA, sW, sC elements after group
 * 0's. bf16 inputs, float32 accumulation. K a multiple of 64; A and W rows
 * 16-byte aligned (bases 16-byte aligned, lda, ldw, sA, sW multiples of 8
 * elements); C aligned to its element size; M, N < 2^31 with fewer than
 * 2^24 tiles of 128 x 128 in C, G <= 65535.
 */
csa_status csa_linear_bf16(const void* A, int64_t lda, int64_t sA, const void* W, int64_t ldw, int64_t sW,
                           void* C, csa_dtype out_t, int64_t ldc, int64_t sC, int64_t M, int64_t N,
                           int64_t K, int64_t G, hipStream_t stream);

/*
 * csa_grouped_out_proj — grouped output projection. The H heads of o
 * [T, H, d] (bf16) form G groups of H/G consecutive heads; group g's
 * concatenated heads [T, (H/G)*d] are projected to rank r by w_group[g]
 * [r, (H/G)*d], the G results concatenated to y [T, G*r] (bf16, in ws) and
 * projected by w_out [D, G*r]:  out [T, D] (bf16) = y * w_out^T.
 * (H/G)*d and G*r multiples of 64. ws: at least
 * csa_grouped_out_proj_workspace_size() bytes, 16-byte aligned.
 */
size_t csa_grouped_out_proj_workspace_size(int64_t T, int32_t G, int32_t r);
csa_status csa_grouped_out_proj(const void* o, const void* w_group, const void* w_out, int64_t T, int32_t H,
                                int32_t d, int32_t G, int32_t r, int32_t D, void* out, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/*
 * csa_query_proj_shared — query projections of the main attention and the
 * lightning indexer from one shared low-rank latent (the indexer shares the
 * main attention's projection): latent [T, r_q] (bf16, in ws) = x [T, D] *
 * w_dq^T (w_dq [r_q, D]); q [T, n_q] = latent * w_uq^T (w_uq [n_q, r_q]);
 * q_idx [T, n_i] = latent * w_iq^T (w_iq [n_i, r_q]); all bf16 (q_idx is
 * quantised for the indexer by csa_quantize_rows). D and r_q multiples of
 * 64. ws: csa_query_proj_shared_workspace_size() bytes.
 */
size_t csa_query_proj_shared_workspace_size(int64_t T, int32_t r_q);
csa_status csa_query_proj_shared(const void* x, const void* w_dq, const void* w_uq, const void* w_iq,
                                 int64_t T, int32_t D, int32_t r_q, int32_t n_q, int32_t n_i, void* q,
                                 void* q_idx, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * csa_kv_proj — the compressor's input streams from the hidden state (the
 * KV and gate projections in front of the compressor; cf-1.com write-up
 * §3.1 builds the compressed entries from per-token KV vectors and gate
 * logits of the two overlapped streams, §3.4 has the indexer's keys built
 * the same way): streams[s] [T, width] = x [T, D] * w[s]^T for s <
 * n_streams, w [n_streams, width, D] (bf16, one linear layer's weight per
 * stream), streams [n_streams, T, width] of out_t (CSA_BF16 or CSA_F32),
 * stream s starting s * T * width elements in. For csa_compress the four
 * streams are C_a, C_b, Z_a, Z_b (n_streams 4, width 128 or the indexer's
 * d_I); rows of several sequences [B, T] are T = B * T rows. D a multiple of
 * 64; x and w 16-byte aligned. No workspace.
 */
csa_status csa_kv_proj(const void* x, const void* w, int64_t T, int32_t D, int32_t n_streams, int32_t width,
                       void* streams, csa_dtype out_t, hipStream_t stream);

/*
 * sparse_attn_bwd — gradients of sparse_attn_fwd (cf-1.com write-up §4.3:
 * training runs a deterministic attention backward; the formulas are the
 * derivatives of the forward's definition above). With P_i = e^{l_i - lse_h},
 * D_h = dO_h . o_h, dP_i = dO_h . K_i and dl_i = P_i (dP_i - D_h):
 *     dq_h    = scale sum_i dl_i K_i,
 *     dK_i   += sum over heads and queries of (scale dl_i q_h + P_i dO_h)
 *              (each key row is both key and value),
 *     dsink_h = -sum over queries of e^{sink_h - lse_h} D_h.
 * Inputs are those of the forward plus its outputs:
 *   out, dout  [B, Tq, H, d] of t: the forward output and its gradient
 *   lse        float32 [B, Tq, H]: the forward's log-sum-exp (sink included)
 * Outputs (all written, including rows no query touches):
 *   dq         [B, Tq, H, d] of t
 *   dkv        float32 [B, N, d];  dx_win float32 [B, T_win, d]
 *   dsink      float32 [H] (summed over B and Tq), or NULL when sink is NULL
 * Limits: t == CSA_BF16, H 64 or 128, d == 128, 1 <= k <= 4096, scale as in
 * the forward, B*Tq < 2^31, B*(N + T_win) < 2^31; idx rows as indexer_topk writes them
 * (an entry repeated within a row is counted once per occurrence).
 * Deterministic: every sum runs in a fixed order that depends only on the
 * shapes (no floating-point atomics), so repeated calls give identical bits.
 * The workspace holds the per-(query, key) gradient rows of up to 4 GiB of
 * query rows at a time (query rows are processed in passes).
 */
size_t sparse_attn_bwd_workspace_size(int64_t B, int64_t Tq, int64_t N, int64_t T_win, int32_t H,
                                      int32_t d, int32_t k, int32_t window);
csa_status sparse_attn_bwd(const void* q, const void* kv, const int32_t* idx, const void* x_win,
                           const int32_t* win_start, const float* sink, const int32_t* q_pos,
                           csa_dtype t, int64_t B, int64_t Tq, int64_t N, int64_t T_win,
                           int32_t H, int32_t d, int32_t k, int32_t window, float scale,
                           const void* out, const float* lse, const void* dout, void* dq,
                           float* dkv, float* dx_win, float* dsink, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/*
 * dense_compressed_attn_bwd — gradients of dense_compressed_attn_fwd
 * (cf-1.com write-up §3.2, §4.3): sparse_attn_bwd with the key set of every
 * query being all visible entries j < n(p) plus its window rows. Same
 * layouts, limits and determinism; ratio >= 1 defines n(p).
 */
size_t dense_attn_bwd_workspace_size(int64_t B, int64_t Tq, int64_t N, int64_t T_win, int32_t H,
                                     int32_t d, int32_t window);
csa_status dense_compressed_attn_bwd(const void* q, const void* kv, const void* x_win,
                                     const int32_t* win_start, const float* sink,
                                     const int32_t* q_pos, csa_dtype t, int64_t B, int64_t Tq,
                                     int64_t N, int64_t T_win, int32_t H, int32_t d, int32_t ratio,
                                     int32_t window, float scale, const void* out, const float* lse,
                                     const void* dout, void* dq, float* dkv, float* dx_win,
                                     float* dsink, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA_HIP_H */
