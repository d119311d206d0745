// Gated KV compressors (CSA 4:1 overlapped two-stream, HCA 128:1 single
// stream) and the row quantiser for the low-precision indexer.
//
// cf-1.com write-up §3.1: CSA merges two independent KV streams with
// softmax-normalised gate weights, adjacent blocks sharing tokens (overlap),
// 4 tokens per entry. §3.2: HCA makes one entry per 128 tokens. §3.4/§4.4:
// the indexer QK path runs in FP4 (OCP MX e2m1 here) or FP8 (e4m3).
//
// These kernels stream HBM: every input byte is read once (CSA reads stream B
// of block j-1 for entry j; the gate logits are re-read from cache for the
// second softmax pass). The bound is HBM bandwidth; one thread owns 8
// channels so each load is 16 B (bf16) or 32 B (f32), and the lanes of one
// entry cover a contiguous row.
#include "common.hpp"

namespace csa {

template <typename TI>
__device__ __forceinline__ void rowmax8(const TI* z, float* m) {
  float v[8];
  Elem<TI>::load8(z, v);
#pragma unroll
  for (int k = 0; k < 8; ++k) m[k] = fmaxf(m[k], v[k]);
}

template <typename TI>
__device__ __forceinline__ void accum8(const TI* z, const TI* c, const float* m, float* s, float* acc) {
  float zv[8], cv[8];
  Elem<TI>::load8(z, zv);
  Elem<TI>::load8(c, cv);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float p = __expf(zv[k] - m[k]);
    s[k] += p;
    acc[k] = fmaf(p, cv[k], acc[k]);
  }
}

// Quantise the 8 values this lane owns, as part of a row of `width` values
// spread over consecutive lanes (lanes_per_row = width / 8, a power of two).
// OUT: CSA_FP8_E4M3 writes 8 code bytes + (first lane) the row's float32
// scale; CSA_FP4_E2M1 writes 4 packed bytes + (first lane of each 4) one E8M0
// byte per 32 channels.
template <int OUT, int LPR>
__device__ __forceinline__ void quantize_store(const float* v, int sub, int64_t row, int width,
                                               void* out, void* scale_out, bool active) {
  if constexpr (OUT == CSA_FP8_E4M3) {
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    float sc = amax / 448.0f;
    if (sc == 0.0f) sc = 1.0f;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) lo |= e4m3_encode(v[k] / sc) << (8 * k);
#pragma unroll
    for (int k = 0; k < 4; ++k) hi |= e4m3_encode(v[4 + k] / sc) << (8 * k);
    if (active) {
      *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(out) + row * width + sub * 8) = make_uint2(lo, hi);
      if (sub == 0) reinterpret_cast<float*>(scale_out)[row] = sc;
    }
  } else {
    static_assert(OUT == CSA_FP4_E2M1, "quantised output");
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const int E = mx_exponent(amax);
    const float mul = pow2i(-E);
    uint32_t packed = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) packed |= e2m1_encode(v[k] * mul) << (4 * k);
    if (active) {
      *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(out) + row * (width / 2) + sub * 4) = packed;
      if ((sub & 3) == 0)
        reinterpret_cast<uint8_t*>(scale_out)[row * (width / 32) + sub / 4] = (uint8_t)(E + 127);
    }
  }
}

// Raw copy of 8 elements (16 or 32 bytes).
template <typename TI>
__device__ __forceinline__ void copy8(const TI* src, TI* dst) {
  if constexpr (sizeof(TI) == 2) {
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
  } else {
    reinterpret_cast<float4*>(dst)[0] = reinterpret_cast<const float4*>(src)[0];
    reinterpret_cast<float4*>(dst)[1] = reinterpret_cast<const float4*>(src)[1];
  }
}

template <typename TO>
__device__ __forceinline__ void store_plain(const float* v, int64_t row, int width, int sub, void* out) {
  Elem<TO>::store8(reinterpret_cast<TO*>(out) + row * width + sub * 8, v);
}

// One lane's 8 channels of a CSA entry: one softmax per channel over the
// gate logits of stream A (rows 0..ratio-1) and, when has_b, stream B (rows
// 0..ratio-1 of the previous block); the rows come from accessors returning
// the lane's 8-value pieces (z and c of each row). The batch compressor and
// the decode-time append share this code, so an entry is the same bit for bit
// whichever built it.
// R > 0: the ratio is R (compile time) and every row is loaded before any is
// used (one memory round trip, for the latency-bound single-entry append);
// the arithmetic and its order are the same as with R = 0 (runtime ratio).
template <typename TI, int R, typename ZA, typename CA, typename ZB, typename CB>
__device__ __forceinline__ void csa_entry8(int ratio, bool has_b, ZA zA, CA cA, ZB zB, CB cB, float* v) {
  float m[8], s[8], acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) { m[k] = -INFINITY; s[k] = 0.f; acc[k] = 0.f; }
  if constexpr (R > 0) {
    float za[R][8], ca[R][8], zb[R][8], cb[R][8];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      Elem<TI>::load8(zA(i), za[i]);
      Elem<TI>::load8(cA(i), ca[i]);
      if (has_b) {
        Elem<TI>::load8(zB(i), zb[i]);
        Elem<TI>::load8(cB(i), cb[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int k = 0; k < 8; ++k) m[k] = fmaxf(m[k], za[i][k]);
    if (has_b) {
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int k = 0; k < 8; ++k) m[k] = fmaxf(m[k], zb[i][k]);
    }
    auto acc8 = [&](const float* zv, const float* cv) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float p = __expf(zv[k] - m[k]);
        s[k] += p;
        acc[k] = fmaf(p, cv[k], acc[k]);
      }
    };
#pragma unroll
    for (int i = 0; i < R; ++i) acc8(za[i], ca[i]);
    if (has_b) {
#pragma unroll
      for (int i = 0; i < R; ++i) acc8(zb[i], cb[i]);
    }
  } else {
    for (int i = 0; i < ratio; ++i) rowmax8(zA(i), m);
    if (has_b)
      for (int i = 0; i < ratio; ++i) rowmax8(zB(i), m);
    for (int i = 0; i < ratio; ++i) accum8(zA(i), cA(i), m, s, acc);
    if (has_b)
      for (int i = 0; i < ratio; ++i) accum8(zB(i), cB(i), m, s, acc);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = acc[k] / s[k];
}

// Store one lane's 8 channels of entry row `row` in the output format.
template <int OUT, int LPE>
__device__ __forceinline__ void csa_store8(const float* v, int sub, int64_t row, int width, void* out,
                                           void* out_scale, bool active) {
  if constexpr (OUT == CSA_F32) {
    if (active) store_plain<float>(v, row, width, sub, out);
  } else if constexpr (OUT == CSA_BF16) {
    if (active) store_plain<uint16_t>(v, row, width, sub, out);
  } else {
    quantize_store<OUT, LPE>(v, sub, row, width, out, out_scale, active);   // every lane: it shuffles
  }
}

// One group of W/8 lanes per entry; 256 threads per block.
template <typename TI, int W, int OUT>
__global__ __launch_bounds__(256) void k_csa_compress(const TI* __restrict__ ca, const TI* __restrict__ cb,
                                                      const TI* __restrict__ za, const TI* __restrict__ zb,
                                                      int64_t B, int64_t T, int64_t N, int ratio,
                                                      void* __restrict__ out, void* __restrict__ out_scale) {
  constexpr int LPE = W / 8;
  constexpr int EPB = 256 / LPE;
  const int tid = threadIdx.x;
  const int sub = tid % LPE;
  const int64_t e = (int64_t)blockIdx.x * EPB + tid / LPE;
  const bool active = e < B * N;
  const int64_t b = active ? e / N : 0;
  const int64_t j = active ? e % N : 0;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (active) {
    const int64_t baseA = (b * T + (int64_t)ratio * j) * W + sub * 8;
    const int64_t baseB = baseA - (int64_t)ratio * W;
    auto zA = [&](int i) { return za + baseA + (int64_t)i * W; };
    auto cA = [&](int i) { return ca + baseA + (int64_t)i * W; };
    auto zB = [&](int i) { return zb + baseB + (int64_t)i * W; };
    auto cB = [&](int i) { return cb + baseB + (int64_t)i * W; };
    if (ratio == 4) csa_entry8<TI, 4>(ratio, j > 0, zA, cA, zB, cB, v);
    else csa_entry8<TI, 0>(ratio, j > 0, zA, cA, zB, cB, v);
  }
  csa_store8<OUT, LPE>(v, sub, e, W, out, out_scale, active);
}

// Decode-time append: the new token of each sequence (rows [B, W] of the
// four streams) at absolute position pos[b] goes into the sequence's ring of
// the last 2*ratio tokens (state [B, 2*ratio, 4, W]: c_a, c_b, z_a, z_b at
// slot position % (2*ratio)); when it completes block j = (pos+1)/ratio - 1,
// entry j is computed from the ring (earlier tokens) and the new rows and
// written to row b*N_cap + j of out. The reads touch the 2*ratio - 1 tokens
// before pos, never the slot being written.
template <typename TI, int W, int OUT>
__global__ __launch_bounds__(256) void k_csa_append(const TI* __restrict__ ca, const TI* __restrict__ cb,
                                                    const TI* __restrict__ za, const TI* __restrict__ zb,
                                                    const int32_t* __restrict__ pos, int64_t B, int ratio,
                                                    TI* __restrict__ state, int64_t N_cap, void* __restrict__ out,
                                                    void* __restrict__ out_scale) {
  constexpr int LPE = W / 8;
  constexpr int EPB = 256 / LPE;
  const int tid = threadIdx.x;
  const int sub = tid % LPE;
  const int64_t b = (int64_t)blockIdx.x * EPB + tid / LPE;
  const bool live = b < B;
  const int32_t p = live ? pos[b] : -1;
  const int R2 = 2 * ratio;
  TI* ring = state + (live ? b : 0) * (int64_t)R2 * 4 * W;
  const int64_t j = ((int64_t)p + 1) / ratio - 1;
  const bool emit = p >= 0 && ((int64_t)p + 1) % ratio == 0 && j < N_cap;
  float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (emit) {
    const int64_t nb = b * W + sub * 8;   // the new rows
    auto slot_row = [&](int64_t t, int q) { return ring + ((int64_t)(t % R2) * 4 + q) * W + sub * 8; };
    const int64_t a0 = (int64_t)ratio * j, b0 = a0 - ratio;
    auto zA = [&](int i) { return i == ratio - 1 ? za + nb : slot_row(a0 + i, 2); };
    auto cA = [&](int i) { return i == ratio - 1 ? ca + nb : slot_row(a0 + i, 0); };
    auto zB = [&](int i) { return slot_row(b0 + i, 3); };
    auto cB = [&](int i) { return slot_row(b0 + i, 1); };
    if (ratio == 4) csa_entry8<TI, 4>(ratio, j > 0, zA, cA, zB, cB, v);
    else csa_entry8<TI, 0>(ratio, j > 0, zA, cA, zB, cB, v);
  }
  csa_store8<OUT, LPE>(v, sub, b * N_cap + (emit ? j : 0), W, out, out_scale, emit);
  if (live && p >= 0) {
    const int64_t nb = b * W + sub * 8;
    TI* dst = ring + (int64_t)(p % R2) * 4 * W + sub * 8;
    copy8(ca + nb, dst);
    copy8(cb + nb, dst + W);
    copy8(za + nb, dst + 2 * W);
    copy8(zb + nb, dst + 3 * W);
  }
}

// One HCA entry computed by a block of 256 threads: W/8 lanes per row,
// 256/(W/8) row slots; pass 1 finds the per-channel max over the rows, pass 2
// sums exp-weights; rows come from accessors (z and c of row i, the lane's 8
// values). Threads tid < W return channel tid of the entry (others 0). Shared
// by the batch compressor and the decode-time append (same bits).
template <typename TI, int W, int R, typename ZR, typename CR>
__device__ __forceinline__ float hca_entry(int ratio, ZR zrow, CR crow, float (*red)[W + 1], float (*red2)[W + 1],
                                           float* mx) {
  constexpr int LPR = W / 8;
  constexpr int RS = 256 / LPR;
  // R > 0: ratio R (compile time, a multiple of RS); each thread loads its
  // R / RS rows up front (same arithmetic, same order)
  constexpr int RPT = R > 0 ? R / RS : 1;
  static_assert(R == 0 || R % RS == 0, "rows split evenly over the row slots");
  const int tid = threadIdx.x;
  const int sub = tid % LPR, slot = tid / LPR;
  float m[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) m[k] = -INFINITY;
  float zr[RPT][8], cr[RPT][8];
  if constexpr (R > 0) {
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      Elem<TI>::load8(zrow(slot + u * RS), zr[u]);
      Elem<TI>::load8(crow(slot + u * RS), cr[u]);
    }
#pragma unroll
    for (int u = 0; u < RPT; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) m[k] = fmaxf(m[k], zr[u][k]);
  } else {
    for (int i = slot; i < ratio; i += RS) rowmax8(zrow(i), m);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) red[slot][sub * 8 + k] = m[k];
  __syncthreads();
  if (tid < W) {
    float a = -INFINITY;
    for (int r = 0; r < RS; ++r) a = fmaxf(a, red[r][tid]);
    mx[tid] = a;
  }
  __syncthreads();
  float s[8], acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) { m[k] = mx[sub * 8 + k]; s[k] = 0.f; acc[k] = 0.f; }
  if constexpr (R > 0) {
#pragma unroll
    for (int u = 0; u < RPT; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float p = __expf(zr[u][k] - m[k]);
        s[k] += p;
        acc[k] = fmaf(p, cr[u][k], acc[k]);
      }
  } else {
    for (int i = slot; i < ratio; i += RS) accum8(zrow(i), crow(i), m, s, acc);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 8; ++k) { red[slot][sub * 8 + k] = s[k]; red2[slot][sub * 8 + k] = acc[k]; }
  __syncthreads();
  float v = 0.f;
  if (tid < W) {
    float ss = 0.f, aa = 0.f;
    for (int r = 0; r < RS; ++r) { ss += red[r][tid]; aa += red2[r][tid]; }
    v = aa / ss;
  }
  return v;
}

template <typename TO>
__device__ __forceinline__ void store1(TO* out, int64_t i, float v) {
  if constexpr (sizeof(TO) == 4) out[i] = v;
  else out[i] = f32_to_bf16(v);
}

// One block per entry.
template <typename TI, typename TO, int W>
__global__ __launch_bounds__(256) void k_hca_compress(const TI* __restrict__ c, const TI* __restrict__ z,
                                                      int64_t T, int64_t N, int ratio, TO* __restrict__ out) {
  constexpr int RS = 256 / (W / 8);
  __shared__ float red[RS][W + 1];
  __shared__ float red2[RS][W + 1];
  __shared__ float mx[W];
  const int sub = threadIdx.x % (W / 8);
  const int64_t e = blockIdx.x;       // entry over B*N
  const int64_t b = e / N, j = e % N;
  const int64_t base = (b * T + (int64_t)ratio * j) * W + sub * 8;
  auto zr = [&](int i) { return z + base + (int64_t)i * W; };
  auto cr = [&](int i) { return c + base + (int64_t)i * W; };
  const float v = ratio == 128 ? hca_entry<TI, W, 128>(ratio, zr, cr, red, red2, mx)
                               : hca_entry<TI, W, 0>(ratio, zr, cr, red, red2, mx);
  if (threadIdx.x < W) store1(out, e * W + threadIdx.x, v);
}

// Decode-time append, one block per sequence: the new token (rows [B, W] of c
// and z) at absolute position pos[b] goes into the sequence's ring of the
// last ratio tokens (state [B, ratio, 2, W]: c, z at slot position % ratio);
// when it completes block j = (pos+1)/ratio - 1, entry j is computed from the
// ring (the block's first ratio - 1 tokens, slot = row) and the new rows and
// written to row b*N_cap + j of out.
template <typename TI, typename TO, int W>
__global__ __launch_bounds__(256) void k_hca_append(const TI* __restrict__ c, const TI* __restrict__ z,
                                                    const int32_t* __restrict__ pos, int ratio,
                                                    TI* __restrict__ state, int64_t N_cap, TO* __restrict__ out) {
  constexpr int RS = 256 / (W / 8);
  __shared__ float red[RS][W + 1];
  __shared__ float red2[RS][W + 1];
  __shared__ float mx[W];
  const int sub = threadIdx.x % (W / 8);
  const int64_t b = blockIdx.x;
  const int32_t p = pos[b];
  if (p < 0) return;   // uniform
  TI* ring = state + b * (int64_t)ratio * 2 * W;
  const int64_t j = ((int64_t)p + 1) / ratio - 1;
  if (((int64_t)p + 1) % ratio == 0 && j < N_cap) {   // uniform
    const int64_t nb = b * W + sub * 8;
    auto zr = [&](int i) { return i == ratio - 1 ? z + nb : ring + ((int64_t)i * 2 + 1) * W + sub * 8; };
    auto cr = [&](int i) { return i == ratio - 1 ? c + nb : ring + (int64_t)i * 2 * W + sub * 8; };
    const float v = ratio == 128 ? hca_entry<TI, W, 128>(ratio, zr, cr, red, red2, mx)
                                 : hca_entry<TI, W, 0>(ratio, zr, cr, red, red2, mx);
    if (threadIdx.x < W) store1(out, (b * N_cap + j) * W + threadIdx.x, v);
  }
  if (threadIdx.x < W / 8) {
    TI* dst = ring + (int64_t)(p % ratio) * 2 * W + sub * 8;
    copy8(c + b * W + sub * 8, dst);
    copy8(z + b * W + sub * 8, dst + W);
  }
}

// One wave per row; lane owns channels [8*lane + 512*it, +8).
template <typename TI, int OUT>
__global__ __launch_bounds__(256) void k_quantize_rows(const TI* __restrict__ x, int64_t rows, int width,
                                                       void* __restrict__ out, void* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;   // whole wave exits together
  const TI* xr = x + row * width;
  if constexpr (OUT == CSA_FP8_E4M3) {
    float amax = 0.f;
    for (int c0 = lane * 8; c0 < width; c0 += 512) {
      float v[8];
      Elem<TI>::load8(xr + c0, v);
#pragma unroll
      for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    float sc = amax / 448.0f;
    if (sc == 0.0f) sc = 1.0f;
    for (int c0 = lane * 8; c0 < width; c0 += 512) {
      float v[8];
      Elem<TI>::load8(xr + c0, v);
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) lo |= e4m3_encode(v[k] / sc) << (8 * k);
#pragma unroll
      for (int k = 0; k < 4; ++k) hi |= e4m3_encode(v[4 + k] / sc) << (8 * k);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(out) + row * width + c0) = make_uint2(lo, hi);
    }
    if (lane == 0) reinterpret_cast<float*>(scale)[row] = sc;
  } else {
    // width % 32 == 0; the loop bound is uniform across each 4-lane block group.
    for (int base = 0; base < width; base += 512) {
      const int c0 = base + lane * 8;
      const bool act = c0 < width;
      float v[8];
      if (act) Elem<TI>::load8(xr + c0, v);
      else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = 0.f;
      }
      float amax = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
      amax = fmaxf(amax, __shfl_xor(amax, 1));
      amax = fmaxf(amax, __shfl_xor(amax, 2));
      const int E = mx_exponent(amax);
      const float mul = pow2i(-E);
      uint32_t packed = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) packed |= e2m1_encode(v[k] * mul) << (4 * k);
      if (act) {
        *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(out) + row * (width / 2) + c0 / 2) = packed;
        if ((lane & 3) == 0) reinterpret_cast<uint8_t*>(scale)[row * (width / 32) + c0 / 32] = (uint8_t)(E + 127);
      }
    }
  }
}

// ------------------------------------------------------------------ launchers

template <typename TI, int W>
static hipError_t launch_csa_w(const void* ca, const void* cb, const void* za, const void* zb, int64_t B,
                               int64_t T, int64_t N, int ratio, void* out, csa_dtype out_t, void* out_scale,
                               hipStream_t s) {
  constexpr int EPB = 256 / (W / 8);
  const dim3 grid((unsigned)cdiv(B * N, EPB));
  const TI *a = (const TI*)ca, *b = (const TI*)cb, *c = (const TI*)za, *d = (const TI*)zb;
  switch (out_t) {
    case CSA_F32: k_csa_compress<TI, W, CSA_F32><<<grid, 256, 0, s>>>(a, b, c, d, B, T, N, ratio, out, out_scale); break;
    case CSA_BF16: k_csa_compress<TI, W, CSA_BF16><<<grid, 256, 0, s>>>(a, b, c, d, B, T, N, ratio, out, out_scale); break;
    case CSA_FP8_E4M3: k_csa_compress<TI, W, CSA_FP8_E4M3><<<grid, 256, 0, s>>>(a, b, c, d, B, T, N, ratio, out, out_scale); break;
    case CSA_FP4_E2M1: k_csa_compress<TI, W, CSA_FP4_E2M1><<<grid, 256, 0, s>>>(a, b, c, d, B, T, N, ratio, out, out_scale); break;
  }
  return hipGetLastError();
}

hipError_t launch_csa_compress(const void* ca, const void* cb, const void* za, const void* zb, csa_dtype in_t,
                               int64_t B, int64_t T, int width, int ratio, void* out, csa_dtype out_t,
                               void* out_scale, hipStream_t s) {
  const int64_t N = T / ratio;
  if (B * N == 0) return hipSuccess;
  timer_before(CSA_KID_COMPRESS, s);
  hipError_t err;
  if (in_t == CSA_F32)
    err = width == 128 ? launch_csa_w<float, 128>(ca, cb, za, zb, B, T, N, ratio, out, out_t, out_scale, s)
                       : launch_csa_w<float, 64>(ca, cb, za, zb, B, T, N, ratio, out, out_t, out_scale, s);
  else
    err = width == 128 ? launch_csa_w<uint16_t, 128>(ca, cb, za, zb, B, T, N, ratio, out, out_t, out_scale, s)
                       : launch_csa_w<uint16_t, 64>(ca, cb, za, zb, B, T, N, ratio, out, out_t, out_scale, s);
  timer_after(CSA_KID_COMPRESS, s);
  return err;
}

template <typename TI, typename TO>
static void launch_hca_t(const void* c, const void* z, int64_t B, int64_t T, int64_t N, int width, int ratio,
                         void* out, hipStream_t s) {
  const dim3 grid((unsigned)(B * N));
  if (width == 128)
    k_hca_compress<TI, TO, 128><<<grid, 256, 0, s>>>((const TI*)c, (const TI*)z, T, N, ratio, (TO*)out);
  else
    k_hca_compress<TI, TO, 64><<<grid, 256, 0, s>>>((const TI*)c, (const TI*)z, T, N, ratio, (TO*)out);
}

hipError_t launch_hca_compress(const void* c, const void* z, csa_dtype in_t, int64_t B, int64_t T, int width,
                               int ratio, void* out, csa_dtype out_t, hipStream_t s) {
  const int64_t N = T / ratio;
  if (B * N == 0) return hipSuccess;
  timer_before(CSA_KID_HCA_COMPRESS, s);
  if (in_t == CSA_F32) {
    if (out_t == CSA_F32) launch_hca_t<float, float>(c, z, B, T, N, width, ratio, out, s);
    else launch_hca_t<float, uint16_t>(c, z, B, T, N, width, ratio, out, s);
  } else {
    if (out_t == CSA_F32) launch_hca_t<uint16_t, float>(c, z, B, T, N, width, ratio, out, s);
    else launch_hca_t<uint16_t, uint16_t>(c, z, B, T, N, width, ratio, out, s);
  }
  hipError_t err = hipGetLastError();
  timer_after(CSA_KID_HCA_COMPRESS, s);
  return err;
}

template <typename TI, int W>
static void launch_csa_append_w(const void* ca, const void* cb, const void* za, const void* zb, int64_t B, int ratio,
                                const int32_t* pos, void* state, int64_t N_cap, void* out, csa_dtype out_t,
                                void* out_scale, hipStream_t s) {
  constexpr int EPB = 256 / (W / 8);
  const dim3 grid((unsigned)cdiv(B, EPB));
  const TI *a = (const TI*)ca, *b = (const TI*)cb, *c = (const TI*)za, *d = (const TI*)zb;
  TI* st = (TI*)state;
  switch (out_t) {
    case CSA_F32: k_csa_append<TI, W, CSA_F32><<<grid, 256, 0, s>>>(a, b, c, d, pos, B, ratio, st, N_cap, out, out_scale); break;
    case CSA_BF16: k_csa_append<TI, W, CSA_BF16><<<grid, 256, 0, s>>>(a, b, c, d, pos, B, ratio, st, N_cap, out, out_scale); break;
    case CSA_FP8_E4M3: k_csa_append<TI, W, CSA_FP8_E4M3><<<grid, 256, 0, s>>>(a, b, c, d, pos, B, ratio, st, N_cap, out, out_scale); break;
    case CSA_FP4_E2M1: k_csa_append<TI, W, CSA_FP4_E2M1><<<grid, 256, 0, s>>>(a, b, c, d, pos, B, ratio, st, N_cap, out, out_scale); break;
  }
}

hipError_t launch_csa_append(const void* ca, const void* cb, const void* za, const void* zb, csa_dtype in_t,
                             int64_t B, int width, int ratio, const int32_t* pos, void* state, int64_t N_cap,
                             void* out, csa_dtype out_t, void* out_scale, hipStream_t s) {
  if (B == 0) return hipSuccess;
  timer_before(CSA_KID_COMPRESS, s);
  if (in_t == CSA_F32) {
    if (width == 128) launch_csa_append_w<float, 128>(ca, cb, za, zb, B, ratio, pos, state, N_cap, out, out_t, out_scale, s);
    else launch_csa_append_w<float, 64>(ca, cb, za, zb, B, ratio, pos, state, N_cap, out, out_t, out_scale, s);
  } else {
    if (width == 128) launch_csa_append_w<uint16_t, 128>(ca, cb, za, zb, B, ratio, pos, state, N_cap, out, out_t, out_scale, s);
    else launch_csa_append_w<uint16_t, 64>(ca, cb, za, zb, B, ratio, pos, state, N_cap, out, out_t, out_scale, s);
  }
  hipError_t err = hipGetLastError();
  timer_after(CSA_KID_COMPRESS, s);
  return err;
}

template <typename TI, typename TO>
static void launch_hca_append_t(const void* c, const void* z, int64_t B, int width, int ratio, const int32_t* pos,
                                void* state, int64_t N_cap, void* out, hipStream_t s) {
  const dim3 grid((unsigned)B);
  if (width == 128)
    k_hca_append<TI, TO, 128><<<grid, 256, 0, s>>>((const TI*)c, (const TI*)z, pos, ratio, (TI*)state, N_cap, (TO*)out);
  else
    k_hca_append<TI, TO, 64><<<grid, 256, 0, s>>>((const TI*)c, (const TI*)z, pos, ratio, (TI*)state, N_cap, (TO*)out);
}

hipError_t launch_hca_append(const void* c, const void* z, csa_dtype in_t, int64_t B, int width, int ratio,
                             const int32_t* pos, void* state, int64_t N_cap, void* out, csa_dtype out_t,
                             hipStream_t s) {
  if (B == 0) return hipSuccess;
  timer_before(CSA_KID_HCA_COMPRESS, s);
  if (in_t == CSA_F32) {
    if (out_t == CSA_F32) launch_hca_append_t<float, float>(c, z, B, width, ratio, pos, state, N_cap, out, s);
    else launch_hca_append_t<float, uint16_t>(c, z, B, width, ratio, pos, state, N_cap, out, s);
  } else {
    if (out_t == CSA_F32) launch_hca_append_t<uint16_t, float>(c, z, B, width, ratio, pos, state, N_cap, out, s);
    else launch_hca_append_t<uint16_t, uint16_t>(c, z, B, width, ratio, pos, state, N_cap, out, s);
  }
  hipError_t err = hipGetLastError();
  timer_after(CSA_KID_HCA_COMPRESS, s);
  return err;
}

hipError_t launch_quantize_rows(const void* x, csa_dtype in_t, int64_t rows, int width, void* out,
                                csa_dtype out_t, void* scale, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)cdiv(rows, 4));
  timer_before(CSA_KID_QUANTIZE, s);
  if (in_t == CSA_F32) {
    if (out_t == CSA_FP8_E4M3) k_quantize_rows<float, CSA_FP8_E4M3><<<grid, 256, 0, s>>>((const float*)x, rows, width, out, scale);
    else k_quantize_rows<float, CSA_FP4_E2M1><<<grid, 256, 0, s>>>((const float*)x, rows, width, out, scale);
  } else {
    if (out_t == CSA_FP8_E4M3) k_quantize_rows<uint16_t, CSA_FP8_E4M3><<<grid, 256, 0, s>>>((const uint16_t*)x, rows, width, out, scale);
    else k_quantize_rows<uint16_t, CSA_FP4_E2M1><<<grid, 256, 0, s>>>((const uint16_t*)x, rows, width, out, scale);
  }
  hipError_t err = hipGetLastError();
  timer_after(CSA_KID_QUANTIZE, s);
  return err;
}

}  // namespace csa
