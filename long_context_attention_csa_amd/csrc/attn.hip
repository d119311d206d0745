// Core attention of CSA (selected compressed entries) and HCA (all visible
// entries), each joined with the uncompressed sliding window and the sink.
//
// cf-1.com write-up §3.1: CSA attends over the top-k compressed entries;
// §3.2: HCA attends densely over all entries; §3.3: both add a branch over the
// latest 128 uncompressed tokens and a learnable sink term in the softmax
// denominator. yfxerp.com write-up §3: sliding_window 128, attention_sink.
//
// One KV head is shared by all query heads (MQA) and the key vector is also
// the value vector, so each key row is gathered once into LDS and serves both
// contractions. A block handles one query and NW*16 heads (one wave per 16
// heads); it walks its key list in tiles of 64:
//   gather  64 key rows (selected entries via idx, or entries 0..n(p)-1, then
//           window rows) into LDS, row-major for S and transposed for O,
//   S^T = K Q^T      MFMA, A = key rows (16 per tile), B = Q^T in registers,
//   online softmax   per head = per lane column; the sink enters as the
//                    initial running max/denominator (logit sink_h, value 0),
//   O^T += V^T P^T   MFMA, P^T straight from the S^T accumulators: the 8
//                    K-slots of a lane are the 2x4 keys it already holds, and
//                    V^T is read from LDS with the same key permutation.
// bf16: v_mfma_f32_16x16x32_bf16; f32: v_mfma_f32_16x16x4_f32 (8 per 32 keys).
// With few queries (decode) the key list is split across blocks (a fixed
// count from the shapes, never from timing) and the partial (O, max, sum)
// triples are merged in a fixed order, so results are deterministic.
#include "common.hpp"

namespace csa {

constexpr int kKT = 64;            // keys per tile
constexpr int kD = 128;            // head dim

template <typename T> struct AttnTypes;
template <> struct AttnTypes<uint16_t> {
  static constexpr int KP = kD + 8;     // row pitch of the row-major tile (elements)
  static constexpr int VP = kKT + 4;    // row pitch of the transposed tile
};
template <> struct AttnTypes<float> {
  static constexpr int KP = kD + 4;
  static constexpr int VP = kKT + 4;
};

// 8 consecutive K-elements of one lane's MFMA operand.
template <typename T> struct Frag;
template <> struct Frag<uint16_t> {
  i32x4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const i32x4*>(p); }
  __device__ __forceinline__ void store(uint16_t* p) const { *reinterpret_cast<i32x4*>(p) = v; }
  __device__ __forceinline__ void zero() { v = i32x4{0, 0, 0, 0}; }
  __device__ __forceinline__ uint16_t elem(int j) const {
    const uint32_t w = (uint32_t)v[j >> 1];
    return (uint16_t)((j & 1) ? (w >> 16) : (w & 0xffffu));
  }
  // keys {0..3} from p, {4..7} from p + 16
  __device__ __forceinline__ void load_split(const uint16_t* p) {
    const uint2 a = *reinterpret_cast<const uint2*>(p);
    const uint2 b = *reinterpret_cast<const uint2*>(p + 16);
    v = i32x4{(int)a.x, (int)a.y, (int)b.x, (int)b.y};
  }
};
template <> struct Frag<float> {
  float v[8];
  __device__ __forceinline__ void load(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ void store(float* p) const {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.f;
  }
  __device__ __forceinline__ float elem(int j) const { return v[j]; }
  __device__ __forceinline__ void load_split(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 16);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

// acc += A(16 x 32) * B(32 x 16) with the 8 K-elements per lane of each fragment.
__device__ __forceinline__ f32x4 mma8(const Frag<uint16_t>& a, const Frag<uint16_t>& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v), __builtin_bit_cast(bf16x8, b.v),
                                                 acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma8(const Frag<float>& a, const Frag<float>& b, f32x4 acc) {
#pragma unroll
  for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[t], b.v[t], acc, 0, 0, 0);
  return acc;
}

template <typename T, bool SPARSE, int NW>
__global__ __launch_bounds__(NW * 64) void k_attn(
    const T* __restrict__ q, const T* __restrict__ kv, const int32_t* __restrict__ idx, const T* __restrict__ x_win,
    const int32_t* __restrict__ win_start, const float* __restrict__ sink, const int32_t* __restrict__ q_pos,
    int64_t Tq, int64_t N, int64_t T_win, int H, int k, int window, int ratio, float scale, int S,
    T* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int KP = AttnTypes<T>::KP, VP = AttnTypes<T>::VP;
  constexpr int NT = NW * 64;
  __shared__ __align__(16) T Kt[kKT * KP];
  __shared__ __align__(16) T Vt[kD * VP];
  __shared__ int valid[kKT];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int64_t r = blockIdx.x;
  const int hg = blockIdx.y / S, sp = blockIdx.y % S;
  const int64_t b = r / Tq;
  const int64_t p = q_pos[r];
  const int64_t n_sel = SPARSE ? (int64_t)k : visible(p, ratio, N);
  const int64_t w0 = win_start[b];
  int64_t lo = p - window + 1;
  if (lo < 0) lo = 0;
  if (lo < w0) lo = w0;
  int64_t hi = p;
  if (hi > w0 + T_win - 1) hi = w0 + T_win - 1;
  const int64_t n_win = (window > 0 && hi >= lo) ? hi - lo + 1 : 0;
  const int64_t nk = n_sel + n_win;
  const int64_t chunk = (nk + S - 1) / S;
  const int64_t kbeg = (int64_t)sp * chunk;
  const int64_t kend = (kbeg + chunk) < nk ? (kbeg + chunk) : nk;

  const int head = hg * (NW * 16) + wv * 16 + col;
  // Q^T fragments (B operand of S^T): lane holds q[head, 32ks + 8g .. +8].
  Frag<T> qf[kD / 32];
  {
    const T* qrow = q + (r * H + head) * kD;
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) qf[ks].load(qrow + 32 * ks + 8 * g);
  }
  const bool has_sink = (sink != nullptr) && sp == 0;
  float m = has_sink ? sink[head] : -INFINITY;
  float lsum = (has_sink && g == 0) ? 1.f : 0.f;
  f32x4 O[kD / 16];
#pragma unroll
  for (int db = 0; db < kD / 16; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t t0 = kbeg; t0 < kend; t0 += kKT) {
    const int nt = (int)((kend - t0) < kKT ? (kend - t0) : kKT);
    // ---- gather: 64 rows x 16 pieces of 8 elements
    for (int c = tid; c < kKT * (kD / 8); c += NT) {
      const int kr = c >> 4, cc = c & 15;
      const int64_t i = t0 + kr;
      const T* src = nullptr;
      if (kr < nt) {
        if (i < n_sel) {
          const int64_t e = SPARSE ? (int64_t)idx[r * k + i] : i;
          if (e >= 0 && e < N) src = kv + (b * N + e) * kD;
        } else {
          src = x_win + (b * T_win + (lo + (i - n_sel) - w0)) * kD;
        }
      }
      Frag<T> v;
      if (src) v.load(src + 8 * cc);
      else v.zero();
      v.store(&Kt[kr * KP + 8 * cc]);
#pragma unroll
      for (int j = 0; j < 8; ++j) Vt[(8 * cc + j) * VP + kr] = v.elem(j);
      if (cc == 0) valid[kr] = src != nullptr;
    }
    __syncthreads();

    // ---- S^T = K Q^T for 4 blocks of 16 keys
    float s[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const T* krow = &Kt[(16 * kb + col) * KP + 8 * g];
#pragma unroll
      for (int ks = 0; ks < kD / 32; ++ks) {
        Frag<T> a;
        a.load(krow + 32 * ks);
        acc = mma8(a, qf[ks], acc);
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = 16 * kb + 4 * g + rr;
        s[kb][rr] = (key < nt && valid[key]) ? acc[rr] * scale : -INFINITY;
      }
    }
    // ---- online softmax (per head = per column)
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) tmax = fmaxf(tmax, s[kb][rr]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mnew = fmaxf(m, tmax);
    const bool live = mnew != -INFINITY;
    const float alpha = live ? __expf(m - mnew) : 1.f;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float pv = live ? __expf(s[kb][rr] - mnew) : 0.f;
        s[kb][rr] = pv;
        psum += pv;
      }
    lsum = fmaf(lsum, alpha, psum);
    m = mnew;
#pragma unroll
    for (int db = 0; db < kD / 16; ++db) O[db] *= alpha;

    // ---- O^T += V^T P^T, two groups of 32 keys. K-slot t of lane group g is
    // key 4g+t (t < 4) or 16+4g+(t-4) (t >= 4) of the group.
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      Frag<T> pf;
      if constexpr (sizeof(T) == 2) {
        pf.v[0] = (int)pack_bf16x2(s[2 * grp][0], s[2 * grp][1]);
        pf.v[1] = (int)pack_bf16x2(s[2 * grp][2], s[2 * grp][3]);
        pf.v[2] = (int)pack_bf16x2(s[2 * grp + 1][0], s[2 * grp + 1][1]);
        pf.v[3] = (int)pack_bf16x2(s[2 * grp + 1][2], s[2 * grp + 1][3]);
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) pf.v[t] = s[2 * grp + (t >> 2)][t & 3];
      }
#pragma unroll
      for (int db = 0; db < kD / 16; ++db) {
        Frag<T> va;
        va.load_split(&Vt[(16 * db + col) * VP + 32 * grp + 4 * g]);
        O[db] = mma8(va, pf, O[db]);
      }
    }
    __syncthreads();
  }

  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (S == 1) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    T* orow = out + (r * H + head) * kD;
#pragma unroll
    for (int db = 0; db < kD / 16; ++db) {
      const float v[4] = {O[db][0] * inv, O[db][1] * inv, O[db][2] * inv, O[db][3] * inv};
      Elem<T>::store4(orow + 16 * db + 4 * g, v);
    }
    if (lse && g == 0) lse[r * H + head] = lsum > 0.f ? m + __logf(lsum) : -INFINITY;
  } else {
    const int64_t pi = (r * H + head) * S + sp;
    float* po = part_o + pi * kD;
#pragma unroll
    for (int db = 0; db < kD / 16; ++db)
      *reinterpret_cast<float4*>(po + 16 * db + 4 * g) = make_float4(O[db][0], O[db][1], O[db][2], O[db][3]);
    if (g == 0) {
      part_ml[2 * pi] = m;
      part_ml[2 * pi + 1] = lsum;
    }
  }
}

// Merge of S partial results per (row, head), in split order. 256 threads =
// 2 (row, head) pairs x 128 channels.
template <typename T>
__global__ __launch_bounds__(256) void k_attn_merge(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                                    int64_t RH, int S, T* __restrict__ out, float* __restrict__ lse) {
  const int64_t rh = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);
  const int d = threadIdx.x & 127;
  if (rh >= RH) return;
  float mx = -INFINITY;
  for (int sp = 0; sp < S; ++sp) mx = fmaxf(mx, part_ml[2 * (rh * S + sp)]);
  float l = 0.f, o = 0.f;
  if (mx != -INFINITY) {
    for (int sp = 0; sp < S; ++sp) {
      const float f = __expf(part_ml[2 * (rh * S + sp)] - mx);
      l = fmaf(part_ml[2 * (rh * S + sp) + 1], f, l);
      o = fmaf(part_o[(rh * S + sp) * kD + d], f, o);
    }
  }
  const float v = l > 0.f ? o / l : 0.f;
  if constexpr (sizeof(T) == 4) out[rh * kD + d] = v;
  else out[rh * kD + d] = f32_to_bf16(v);
  if (lse && d == 0) lse[rh] = l > 0.f ? mx + __logf(l) : -INFINITY;
}

// ------------------------------------------------------------------ host side

static int pick_nw(int H) {
  const int hb = H / 16;
  return (hb % 4 == 0) ? 4 : (hb % 2 == 0 ? 2 : 1);
}

int attn_splits(int64_t rows, int H, int64_t nk_max) {
  const int nw = pick_nw(H);
  const int64_t base = rows * (H / (16 * nw));
  if (base >= 256) return 1;
  int64_t s = cdiv(512, base);
  const int64_t by_keys = nk_max / 128 > 1 ? nk_max / 128 : 1;
  if (s > by_keys) s = by_keys;
  if (s > 64) s = 64;
  return (int)(s < 1 ? 1 : s);
}

size_t attn_ws_bytes(int64_t rows, int H, int64_t nk_max) {
  const int S = attn_splits(rows, H, nk_max);
  if (S == 1) return 0;
  return (size_t)rows * H * S * (kD + 2) * 4;
}

template <typename T, bool SPARSE, int NW>
static void launch_attn_t(dim3 grid, hipStream_t st, const void* q, const void* kv, const int32_t* idx,
                          const void* x_win, const int32_t* win_start, const float* sink, const int32_t* q_pos,
                          int64_t Tq, int64_t N, int64_t T_win, int H, int k, int window, int ratio, float scale,
                          int S, void* out, float* lse, float* po, float* pml) {
  k_attn<T, SPARSE, NW><<<grid, NW * 64, 0, st>>>((const T*)q, (const T*)kv, idx, (const T*)x_win, win_start, sink,
                                                  q_pos, Tq, N, T_win, H, k, window, ratio, scale, S, (T*)out, lse,
                                                  po, pml);
}

template <typename T, bool SPARSE>
static void launch_attn_nw(int nw, dim3 grid, hipStream_t st, const void* q, const void* kv, const int32_t* idx,
                           const void* x_win, const int32_t* win_start, const float* sink, const int32_t* q_pos,
                           int64_t Tq, int64_t N, int64_t T_win, int H, int k, int window, int ratio, float scale,
                           int S, void* out, float* lse, float* po, float* pml) {
  if (nw == 4) launch_attn_t<T, SPARSE, 4>(grid, st, q, kv, idx, x_win, win_start, sink, q_pos, Tq, N, T_win, H, k, window, ratio, scale, S, out, lse, po, pml);
  else if (nw == 2) launch_attn_t<T, SPARSE, 2>(grid, st, q, kv, idx, x_win, win_start, sink, q_pos, Tq, N, T_win, H, k, window, ratio, scale, S, out, lse, po, pml);
  else launch_attn_t<T, SPARSE, 1>(grid, st, q, kv, idx, x_win, win_start, sink, q_pos, Tq, N, T_win, H, k, window, ratio, scale, S, out, lse, po, pml);
}

hipError_t launch_attention(bool sparse, csa_dtype t, const void* q, const void* kv, const int32_t* idx,
                            const void* x_win, const int32_t* win_start, const float* sink, const int32_t* q_pos,
                            int64_t B, int64_t Tq, int64_t N, int64_t T_win, int H, int k, int window, int ratio,
                            float scale, void* out, float* lse, void* ws, int64_t nk_max, hipStream_t st) {
  const int64_t rows = B * Tq;
  if (rows == 0) return hipSuccess;
  const int nw = pick_nw(H);
  const int S = attn_splits(rows, H, nk_max);
  float* po = reinterpret_cast<float*>(ws);
  float* pml = po ? po + (size_t)rows * H * S * kD : nullptr;
  const dim3 grid((unsigned)rows, (unsigned)((H / (16 * nw)) * S));
  const int kid = sparse ? CSA_KID_SPARSE_ATTN : CSA_KID_DENSE_ATTN;
  timer_before(kid, st);
  if (t == CSA_BF16) {
    if (sparse) launch_attn_nw<uint16_t, true>(nw, grid, st, q, kv, idx, x_win, win_start, sink, q_pos, Tq, N, T_win, H, k, window, ratio, scale, S, out, lse, po, pml);
    else launch_attn_nw<uint16_t, false>(nw, grid, st, q, kv, idx, x_win, win_start, sink, q_pos, Tq, N, T_win, H, k, window, ratio, scale, S, out, lse, po, pml);
  } else {
    if (sparse) launch_attn_nw<float, true>(nw, grid, st, q, kv, idx, x_win, win_start, sink, q_pos, Tq, N, T_win, H, k, window, ratio, scale, S, out, lse, po, pml);
    else launch_attn_nw<float, false>(nw, grid, st, q, kv, idx, x_win, win_start, sink, q_pos, Tq, N, T_win, H, k, window, ratio, scale, S, out, lse, po, pml);
  }
  hipError_t e = hipGetLastError();
  timer_after(kid, st);
  if (e != hipSuccess || S == 1) return e;
  const int64_t RH = rows * H;
  timer_before(CSA_KID_ATTN_MERGE, st);
  if (t == CSA_BF16) k_attn_merge<uint16_t><<<dim3((unsigned)cdiv(RH, 2)), 256, 0, st>>>(po, pml, RH, S, (uint16_t*)out, lse);
  else k_attn_merge<float><<<dim3((unsigned)cdiv(RH, 2)), 256, 0, st>>>(po, pml, RH, S, (float*)out, lse);
  e = hipGetLastError();
  timer_after(CSA_KID_ATTN_MERGE, st);
  return e;
}

}  // namespace csa
