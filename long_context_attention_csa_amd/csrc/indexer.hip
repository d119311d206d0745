// Lightning indexer: scores I(p,s) = sum_h w(p,h) * ReLU(q(p,h) . k(s)) and
// exact per-query top-k over the compressed entries.
//
// cf-1.com write-up §3.1: each query picks its top-k compressed entries through
// the lightning indexer; §3.4: the indexer is low-rank and low-precision, its
// QK runs in FP4; §2.4: k = 512 (Flash) or 1024 (Pro). yfxerp.com write-up §3:
// top_k_blocks 1024, indexer_rank 64.
//
// Score stage (k_index_score). The QK contraction is a dense GEMM (heads x
// entries per query), so it runs on MFMA:
//   fp8 / fp4  v_mfma_scale_f32_16x16x128_f8f6f4 (K = 128 per instruction;
//              fp4 uses the hardware E8M0 block scales, fp8 uses unit block
//              scales and folds the per-row float32 scales in afterwards:
//              ReLU commutes with a positive factor),
//   bf16       v_mfma_f32_16x16x32_bf16,
//   f32        v_mfma_f32_16x16x4_f32.
// Layout: A = query heads (16 per block, the row index), B = 16 entries (the
// column index). Each lane of a wave owns one entry (lane % 16) and one group
// of 4 heads (lane / 16) of the 16x16 result, so the weighted ReLU head sum is
// in-register plus two cross-lane adds. Keys are read straight from HBM into
// B-operand registers: every lane reads a contiguous 16-32 B piece and the 64
// lanes of one load cover 16 whole key rows, i.e. the scan is one coalesced
// stream. Up to 4 consecutive queries of one sequence share each key load.
//
// Select stage (k_topk_select, one block per query row). The score kernel
// also writes the maximum of every group of 16 consecutive entries. The k-th
// largest group maximum tau is a lower bound of the k-th largest score (at
// least k groups hold an entry >= tau), so the top-k lies among the entries
// >= tau, which are read only from groups whose maximum is >= tau. On random
// scores that is about k candidates out of n. They are resolved exactly by a
// radix select on 64-bit (order-preserving score key, inverted index)
// composites, which realises the total order "score descending, index
// ascending"; each chosen index is written at its rank among the chosen.
// Rows with few groups per selected entry, and candidate sets too large for
// LDS (heavy ties), take the full-row path: a 13-bit histogram over all
// scores, then the same exact radix select on the boundary bucket.
// Deterministic by construction (atomics only build sets, never orders).
#include "common.hpp"

#include <type_traits>

namespace csa {

constexpr int kTopkThreads = 1024;
constexpr int kHistBits = 13;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kCandCap = 8192;            // candidates held in LDS
constexpr int kMaxK = 2048;
constexpr int kGroup = 16;                // entries per group maximum
constexpr int kGroupFactor = 2;           // group path when groups >= 2k

// ------------------------------------------------------------------ score storage
// Scores are stored as float32, or (the bf16-score variant) as bf16: the
// float32 score rounded to nearest even once, before anything uses it, so
// group maxima, stored scores and the selection all see the same value.
template <typename SC> struct ScoreT;
template <> struct ScoreT<float> {
  __device__ __forceinline__ static float round(float v) { return v; }
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct ScoreT<uint16_t> {
  __device__ __forceinline__ static float round(float v) { return __uint_as_float((uint32_t)f32_to_bf16(v) << 16); }
  __device__ __forceinline__ static float load(const uint16_t* p, int64_t i) { return __uint_as_float((uint32_t)p[i] << 16); }
  __device__ __forceinline__ static void store(uint16_t* p, int64_t i, float v) {
    p[i] = (uint16_t)(__float_as_uint(v) >> 16);   // v is already a bf16 value
  }
};
// 8 consecutive scores from a 16-byte aligned address (float: two float4
// loads, bf16: one).
template <typename SC>
__device__ __forceinline__ void load_scores8(const SC* p, float* v) {
  if constexpr (sizeof(SC) == 4) {
    const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
}

// ------------------------------------------------------------------ operand loads
// Per-format A/B operand of one 16x16 MFMA tile, for one lane:
//   row/col index = lane % 16, K-group g = lane / 16.
template <int FMT, int DI> struct Operand;

template <int DI> struct Operand<CSA_FP8_E4M3, DI> {
  i32x8 v;
  __device__ __forceinline__ void load(const uint8_t* row, int g) {
    if (DI == 128 || g < 2) {
      const i32x4 a = *reinterpret_cast<const i32x4*>(row + 32 * g);
      const i32x4 b = *reinterpret_cast<const i32x4*>(row + 32 * g + 16);
      v = i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    } else {
      v = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
};

template <int DI> struct Operand<CSA_FP4_E2M1, DI> {
  i32x4 v;      // 32 e2m1 values; the MFMA reads only the low 4 dwords of its operand
  int scale;
  __device__ __forceinline__ void load(const uint8_t* row, const uint8_t* srow, int g) {
    if (DI == 128 || g < 2) {
      v = *reinterpret_cast<const i32x4*>(row + 16 * g);
      scale = srow[g];
    } else {
      v = i32x4{0, 0, 0, 0};
      scale = 127;
    }
  }
};

template <int DI> struct Operand<CSA_BF16, DI> {
  bf16x8 v[DI / 32];
  __device__ __forceinline__ void load(const uint16_t* row, int g) {
#pragma unroll
    for (int ks = 0; ks < DI / 32; ++ks)
      v[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(row + 32 * ks + 8 * g));
  }
};

template <int DI> struct Operand<CSA_F32, DI> {
  float v[DI / 32][8];
  __device__ __forceinline__ void load(const float* row, int g) {
#pragma unroll
    for (int ks = 0; ks < DI / 32; ++ks) {
      const float4 a = *reinterpret_cast<const float4*>(row + 32 * ks + 8 * g);
      const float4 b = *reinterpret_cast<const float4*>(row + 32 * ks + 8 * g + 4);
      v[ks][0] = a.x; v[ks][1] = a.y; v[ks][2] = a.z; v[ks][3] = a.w;
      v[ks][4] = b.x; v[ks][5] = b.y; v[ks][6] = b.z; v[ks][7] = b.w;
    }
  }
};

template <int FMT, int DI>
__device__ __forceinline__ f32x4 mma_tile(const Operand<FMT, DI>& a, const Operand<FMT, DI>& b) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (FMT == CSA_FP8_E4M3) {
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a.v, b.v, acc, 0, 0, 0, 127, 0, 127);
  } else if constexpr (FMT == CSA_FP4_E2M1) {
    const i32x8 av = {a.v[0], a.v[1], a.v[2], a.v[3], 0, 0, 0, 0};
    const i32x8 bv = {b.v[0], b.v[1], b.v[2], b.v[3], 0, 0, 0, 0};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 4, 4, 0, a.scale, 0, b.scale);
  } else if constexpr (FMT == CSA_BF16) {
#pragma unroll
    for (int ks = 0; ks < DI / 32; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v[ks], b.v[ks], acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int ks = 0; ks < DI / 32; ++ks)
#pragma unroll
      for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[ks][t], b.v[ks][t], acc, 0, 0, 0);
  }
  return acc;
}

template <int FMT> struct Storage { typedef uint8_t type; };
template <> struct Storage<CSA_BF16> { typedef uint16_t type; };
template <> struct Storage<CSA_F32> { typedef float type; };

// Row length in storage units of one d_I vector.
template <int FMT, int DI> __host__ __device__ constexpr int row_units() {
  return FMT == CSA_FP4_E2M1 ? DI / 2 : DI;
}

// ------------------------------------------------------------------ lane reductions
// Sum of the four lanes l, l^16, l^32, l^48 (VALU permlane swaps: each swap
// returns both halves, whose sum pairs every lane with its partner).
__device__ __forceinline__ float sum_xor16_32(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}
// Maximum over the 16 lanes of a row (DPP row rotations).
__device__ __forceinline__ float max_row16(float v) {
  v = fmaxf(v, __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x128, 0xf, 0xf, false)));
  v = fmaxf(v, __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x124, 0xf, 0xf, false)));
  v = fmaxf(v, __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x122, 0xf, 0xf, false)));
  v = fmaxf(v, __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x121, 0xf, 0xf, false)));
  return v;
}

// Wave-wide max / min / inclusive sum on the VALU (DPP row rotations and
// shifts, row broadcasts and permlane swaps; no LDS traffic).
__device__ __forceinline__ float wave_max(float v) {
  v = max_row16(v);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float wave_min(float v) { return -wave_max(-v); }
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// Wave-wide maximum of an unsigned value, in every lane (DPP row rotations,
// then the two permlane swaps across rows).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x128, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x124, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x122, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x121, 0xf, 0xf, false));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max((uint32_t)a[0], (uint32_t)a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((uint32_t)c[0], (uint32_t)c[1]);
}

// Selection composite of entry i with order key `key`: larger composite =
// earlier in the total order (score descending, index ascending); 0 marks
// "no entry" (below every real composite: an order key is never 0 for a
// finite score).
__device__ __forceinline__ unsigned long long composite(uint32_t key, int64_t i) {
  return ((unsigned long long)key << 32) | (unsigned long long)(0xffffffffu - (uint32_t)i);
}
__device__ __forceinline__ int composite_index(unsigned long long c) {
  return (int)(0xffffffffu - (uint32_t)(c & 0xffffffffu));
}

// ------------------------------------------------------------------ score kernel
// grid.x: entry chunk (chunk_entries entries each), grid.y: query group
// (QB consecutive queries of one sequence), 256 threads (4 waves).
// Group gy covers rows row_lo(gy) .. ; row r writes scores at sbase + (r - srow0) * N.
template <int FMT, int DI, int HB, int QB, int UB, bool DBUF, typename SC>
__global__ __launch_bounds__(256) void k_index_score(
    const void* __restrict__ q_idx, const void* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ k_idx, const void* __restrict__ k_scale, const int32_t* __restrict__ q_pos,
    int64_t Tq, int64_t N, int H_I, int ratio, int64_t group0, int64_t groups_per_batch,
    int64_t chunk_entries, SC* __restrict__ sbase, int64_t srow0, float* __restrict__ gbase, int64_t grow0) {
  typedef typename Storage<FMT>::type ST;
  constexpr int RU = row_units<FMT, DI>();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int64_t grp = group0 + blockIdx.y;
  const int64_t b = grp / groups_per_batch;
  const int64_t t0 = (grp % groups_per_batch) * QB;
  const int nq = (int)((Tq - t0) < QB ? (Tq - t0) : QB);

  int64_t nvis[QB];
  int64_t nmax = 0;
#pragma unroll
  for (int qi = 0; qi < QB; ++qi) {
    nvis[qi] = 0;
    if (qi < nq) nvis[qi] = visible(q_pos[b * Tq + t0 + qi], ratio, N);
    nmax = nvis[qi] > nmax ? nvis[qi] : nmax;
  }
  const int64_t e_begin = (int64_t)blockIdx.x * chunk_entries;
  if (e_begin >= nmax) return;
  const int64_t e_end = (e_begin + chunk_entries) < nmax ? (e_begin + chunk_entries) : nmax;

  // Query operands and folded head weights, per query and head block.
  Operand<FMT, DI> qa[QB][HB];
  float wq[QB][HB][4];
#pragma unroll
  for (int qi = 0; qi < QB; ++qi) {
    const int64_t r = b * Tq + t0 + (qi < nq ? qi : 0);
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int hrow = hb * 16 + col;          // A row = head
      const int hsafe = hrow < H_I ? hrow : 0;
      const ST* qrow = reinterpret_cast<const ST*>(q_idx) + (r * H_I + hsafe) * RU;
      if constexpr (FMT == CSA_FP4_E2M1)
        qa[qi][hb].load(qrow, reinterpret_cast<const uint8_t*>(q_scale) + (r * H_I + hsafe) * (DI / 32), g);
      else
        qa[qi][hb].load(qrow, g);
      if (hrow >= H_I) {   // padded head: zero operand
        if constexpr (FMT == CSA_FP8_E4M3) qa[qi][hb].v = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        else if constexpr (FMT == CSA_FP4_E2M1) qa[qi][hb].v = i32x4{0, 0, 0, 0};
        else if constexpr (FMT == CSA_BF16) {
#pragma unroll
          for (int ks = 0; ks < DI / 32; ++ks) qa[qi][hb].v[ks] = __builtin_bit_cast(bf16x8, i32x4{0, 0, 0, 0});
        } else {
#pragma unroll
          for (int ks = 0; ks < DI / 32; ++ks)
#pragma unroll
            for (int t = 0; t < 8; ++t) qa[qi][hb].v[ks][t] = 0.f;
        }
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int h = hb * 16 + 4 * g + rr;    // C row held by this lane
        float wv_ = 0.f;
        if (h < H_I && qi < nq) {
          wv_ = w[r * H_I + h];
          if constexpr (FMT == CSA_FP8_E4M3) wv_ *= reinterpret_cast<const float*>(q_scale)[r * H_I + h];
        }
        wq[qi][hb][rr] = wv_;
      }
    }
  }

  const ST* kbase = reinterpret_cast<const ST*>(k_idx) + b * N * RU;
  const int64_t G = (N + kGroup - 1) / kGroup;
  // Keys are consumed in batches of UB 16-entry blocks per wave (64*UB
  // entries per block-wide batch); with DBUF the loads of batch i+1 are in
  // flight while batch i is computed.
  constexpr int64_t STEP = 64 * UB;
  auto load_batch = [&](Operand<FMT, DI>* kb, float* ks, int64_t base) {
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int64_t e = base + 16 * wv + 64 * u + col;
      const int64_t esafe = e < N ? e : N - 1;
      if constexpr (FMT == CSA_FP4_E2M1)
        kb[u].load(kbase + esafe * RU, reinterpret_cast<const uint8_t*>(k_scale) + (b * N + esafe) * (DI / 32), g);
      else
        kb[u].load(kbase + esafe * RU, g);
      ks[u] = 1.f;
      if constexpr (FMT == CSA_FP8_E4M3) ks[u] = reinterpret_cast<const float*>(k_scale)[b * N + esafe];
    }
  };
  auto compute_batch = [&](const Operand<FMT, DI>* kb, const float* ks, int64_t base) {
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int64_t e0 = base + 16 * wv + 64 * u;
      if (e0 >= e_end) break;
      const int64_t e = e0 + col;
#pragma unroll
      for (int qi = 0; qi < QB; ++qi) {
        if (qi >= nq) break;
        float part = 0.f;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          const f32x4 acc = mma_tile<FMT, DI>(qa[qi][hb], kb[u]);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) part = fmaf(wq[qi][hb][rr], fmaxf(acc[rr], 0.f), part);
        }
        part = sum_xor16_32(part);
        if constexpr (FMT == CSA_FP8_E4M3) part *= ks[u];
        part = ScoreT<SC>::round(part);
        const bool ok = e < nvis[qi];
        // group maximum over the 16 entries of this block (valid entries only)
        const float gm = max_row16(ok ? part : -INFINITY);
        const int64_t r = b * Tq + t0 + qi;
        if (g == 0 && ok) ScoreT<SC>::store(sbase, (r - srow0) * N + e, part);
        if (gbase && lane == 0 && e0 < nvis[qi]) gbase[(r - grow0) * G + e0 / kGroup] = gm;
      }
    }
  };
  if constexpr (DBUF) {
    Operand<FMT, DI> kA[UB], kB[UB];
    float sA[UB], sB[UB];
    load_batch(kA, sA, e_begin);
    for (int64_t base = e_begin; base < e_end; base += 2 * STEP) {
      if (base + STEP < e_end) load_batch(kB, sB, base + STEP);
      compute_batch(kA, sA, base);
      if (base + STEP >= e_end) break;
      if (base + 2 * STEP < e_end) load_batch(kA, sA, base + 2 * STEP);
      compute_batch(kB, sB, base + STEP);
    }
  } else {
    for (int64_t base = e_begin; base < e_end; base += STEP) {
      Operand<FMT, DI> kA[UB];
      float sA[UB];
      load_batch(kA, sA, base);
      compute_batch(kA, sA, base);
    }
  }
}

// ------------------------------------------------------------------ decode score kernel
// One query per block row, quantised keys (fp8 / fp4), d_I = 128: the path
// that streams a whole long-context key cache per query.
//
// Each wave owns NB batches of 64 consecutive entries (4 MFMA tiles of 16);
// batch i of wave w starts at entry chunk + 64 * (w + 4 * i), so the block's
// four waves read 256 contiguous entries per step. Loads of batch i + DEPTH - 1
// are issued before batch i is computed (a register ring of DEPTH batches)
// and every result stays in registers until the loop ends: on gfx9 one
// counter tracks both loads and stores, so a store between prefetched loads
// would make each wait drain the whole pipeline.
//
// After the 4 tiles of a batch, a reduce-scatter over the four lane rows
// (two permlane32 swaps, one permlane16 swap) leaves lane l holding the
// full weighted score of entry base + l: the fp8 entry scale is one
// coalesced dword per lane, the score store is one 256-byte store per batch.
// fp4 block scales are loaded the same way (one word of 4 E8M0 bytes per
// entry, lane l = entry base + l) and transposed across the rows so lane
// (col, g) holds, in byte u, the scale of K-block g of entry 16u + col; the
// MFMA's scale byte select picks byte u for tile u.
// fp8 operands use a K order shared by queries and keys: lane group g holds
// bytes [16g, 16g + 16) and [64 + 16g, 64 + 16g + 16) of a row, so each of the
// two loads of a tile reads 64 contiguous bytes of every entry.

template <int FMT> struct DecBatch;
template <> struct DecBatch<CSA_FP4_E2M1> {
  i32x4 v[4];
  uint32_t sc;           // scale word of entry base + lane
};
template <> struct DecBatch<CSA_FP8_E4M3> {
  i32x4 lo[4], hi[4];
  float sc;              // float32 scale of entry base + lane
};

// max(x, 0) as one integer max on the bit pattern (a set sign bit reads as a
// negative integer; -0 and negatives give +0), free of the NaN-quieting
// canonicalisation a float max carries.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Sum over the four lane rows of tile part[g], delivered to lane (col, g).
__device__ __forceinline__ float reduce_scatter4(float p0, float p1, float p2, float p3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2), false, false);
  const float s0 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3), false, false);
  const float s1 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(s0), __float_as_uint(s1), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// 4x4 byte transpose across the lane rows: in lane (col, r), byte c of the
// input belongs to row c; the result's byte u is byte r of row u's input.
__device__ __forceinline__ uint32_t transpose_rows_bytes(uint32_t w, int lane) {
  const auto a = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  const uint32_t m = __builtin_amdgcn_perm(a[1], a[0], lane < 32 ? 0x05040100u : 0x07060302u);
  const auto b = __builtin_amdgcn_permlane16_swap(m, m, false, false);
  return __builtin_amdgcn_perm(b[1], b[0], ((lane >> 4) & 1) ? 0x07030501u : 0x06020400u);
}

//
// Selection summary (LT > 0, the list mode): instead of group maxima, each
// wave leaves the LT largest selection composites of its 64 * NB entries
// (score key, inverted index; 0 past the visible entries), largest first, at
// lbase + (r - lrow0) * (4 X LT) + (4 x + w) LT. Each lane sorts its NB
// composites; then LT rounds take the wave's largest head (a wave maximum of
// the keys, and of the inverted indices among lanes that tie on the key) and
// the lane that held it moves to its next composite. The top-k selection then
// reads these lists (k_topk_lists) instead of the group maxima.
template <int FMT, int HB, int NB, int DEPTH, int LT, typename SC>
__global__ __launch_bounds__(256) void k_index_score_dec(
    const void* __restrict__ q_idx, const void* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ k_idx, const void* __restrict__ k_scale, const int32_t* __restrict__ q_pos,
    int64_t Tq, int64_t N, int H_I, int ratio, int64_t row_begin, SC* __restrict__ sbase, int64_t srow0,
    float* __restrict__ gbase, int64_t grow0, unsigned long long* __restrict__ lbase, int64_t lrow0) {
  constexpr int DI = 128;
  constexpr int RB = FMT == CSA_FP4_E2M1 ? DI / 2 : DI;    // bytes per key row
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int64_t r = row_begin + blockIdx.y;                  // query row
  const int64_t b = (int64_t)((uint32_t)r / (uint32_t)Tq);   // its sequence (rows < 2^31)
  // Batch i of wave w in block x covers entries 64 * (w + 4 * (x + X * i)) ..
  // + 63 (X = grid width): at step i the whole grid reads one contiguous window.
  const int64_t X = gridDim.x;
  auto batch_base = [&](int i) -> int64_t { return 64 * (wv + 4 * ((int64_t)blockIdx.x + X * i)); };
  const int64_t e_begin = 256 * (int64_t)blockIdx.x;        // the block's first entry

  // The key stream depends only on the block: its first loads are issued
  // before anything else. Each batch addresses from a uniform base (clamped
  // to N - 1) with 32-bit lane offsets; entries past N read entry N - 1 and
  // entries past the query's visible count are masked at the store.
  const uint8_t* krow = reinterpret_cast<const uint8_t*>(k_idx) + b * N * RB;
  const uint8_t* srow_k = reinterpret_cast<const uint8_t*>(k_scale) + b * N * 4;
  auto load = [&](DecBatch<FMT>& d, int i) {
    const int64_t bw = 256 * ((int64_t)blockIdx.x + X * i);   // block's entries this step
    const int64_t bb = bw < N - 1 ? bw : N - 1;               // uniform, <= N - 1
    const uint32_t lim = (uint32_t)(N - 1 - bb < 255 ? N - 1 - bb : 255);
    const uint8_t* kbat = krow + bb * RB;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t e = 64u * wv + 16u * u + (uint32_t)col;
      e = e < lim ? e : lim;
      const uint32_t off = e * RB + 16u * g;
      if constexpr (FMT == CSA_FP4_E2M1) {
        d.v[u] = *reinterpret_cast<const i32x4*>(kbat + off);
      } else {
        d.lo[u] = *reinterpret_cast<const i32x4*>(kbat + off);
        d.hi[u] = *reinterpret_cast<const i32x4*>(kbat + off + 64);
      }
    }
    uint32_t el = 64u * wv + (uint32_t)lane;
    el = el < lim ? el : lim;
    if constexpr (FMT == CSA_FP4_E2M1)
      d.sc = reinterpret_cast<const uint32_t*>(srow_k + bb * 4)[el];
    else
      d.sc = reinterpret_cast<const float*>(srow_k + bb * 4)[el];
  };
  DecBatch<FMT> ring[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH - 1 && i < NB; ++i) load(ring[i], i);

  const int64_t nvis = visible(q_pos[r], ratio, N);
  if (e_begin >= nvis) {             // nothing visible in this chunk (uniform)
    __builtin_amdgcn_s_waitcnt(0);   // drain the prefetched loads before leaving
    return;
  }
  // query operands (A: head = lane % 16 within head block hb) and folded
  // weights; padded heads (>= H_I) read head 0 and are zeroed
  i32x4 qa[HB], qb[HB];
  int qs8[HB];
  float wq[HB][4];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int hrow = hb * 16 + col;
    const bool live = hrow < H_I;
    const int64_t qr = r * H_I + (live ? hrow : 0);
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(q_idx) + qr * RB;
    const i32x4 z = {0, 0, 0, 0};
    qa[hb] = *reinterpret_cast<const i32x4*>(qrow + 16 * g);
    qa[hb] = live ? qa[hb] : z;
    if constexpr (FMT == CSA_FP4_E2M1) {
      const int sc = reinterpret_cast<const uint8_t*>(q_scale)[qr * (DI / 32) + g];
      qs8[hb] = live ? sc : 127;
    } else {
      qb[hb] = *reinterpret_cast<const i32x4*>(qrow + 64 + 16 * g);
      qb[hb] = live ? qb[hb] : z;
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int h = hb * 16 + 4 * g + rr;
      const int hs = h < H_I ? h : 0;
      float wv_ = w[r * H_I + hs];
      if constexpr (FMT == CSA_FP8_E4M3) wv_ *= reinterpret_cast<const float*>(q_scale)[r * H_I + hs];
      wq[hb][rr] = h < H_I ? wv_ : 0.f;
    }
  }

  auto tile = [&](const DecBatch<FMT>& d, uint32_t st, auto U) -> float {
    constexpr int u = decltype(U)::value;
    float part = 0.f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (FMT == CSA_FP4_E2M1) {
        const i32x8 av = {qa[hb][0], qa[hb][1], qa[hb][2], qa[hb][3], 0, 0, 0, 0};
        const i32x8 bv = {d.v[u][0], d.v[u][1], d.v[u][2], d.v[u][3], 0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 4, 4, 0, qs8[hb], u, (int)st);
      } else {
        const i32x8 av = {qa[hb][0], qa[hb][1], qa[hb][2], qa[hb][3], qb[hb][0], qb[hb][1], qb[hb][2], qb[hb][3]};
        const i32x8 bv = {d.lo[u][0], d.lo[u][1], d.lo[u][2], d.lo[u][3], d.hi[u][0], d.hi[u][1], d.hi[u][2], d.hi[u][3]};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) part = fmaf(wq[hb][rr], relu_bits(acc[rr]), part);
    }
    return part;
  };

  float out_s[NB];
  [[maybe_unused]] float out_g[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    __builtin_amdgcn_sched_barrier(0);   // keep the ring: no load hoisted across batches
    if (i + DEPTH - 1 < NB) load(ring[(i + DEPTH - 1) % DEPTH], i + DEPTH - 1);
    const DecBatch<FMT>& d = ring[i % DEPTH];
    uint32_t st = 0;
    if constexpr (FMT == CSA_FP4_E2M1) st = transpose_rows_bytes(d.sc, lane);
    const float p0 = tile(d, st, std::integral_constant<int, 0>{});
    const float p1 = tile(d, st, std::integral_constant<int, 1>{});
    const float p2 = tile(d, st, std::integral_constant<int, 2>{});
    const float p3 = tile(d, st, std::integral_constant<int, 3>{});
    float s = reduce_scatter4(p0, p1, p2, p3);
    if constexpr (FMT == CSA_FP8_E4M3) s *= d.sc;
    s = ScoreT<SC>::round(s);
    out_s[i] = s;
    if constexpr (LT == 0) {
      const bool ok = batch_base(i) + lane < nvis;
      out_g[i] = max_row16(ok ? s : -INFINITY);
    }
  }
  SC* srow = sbase + (r - srow0) * N;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int64_t e0 = batch_base(i);
    if (e0 + lane < nvis) ScoreT<SC>::store(srow, e0 + lane, out_s[i]);
  }
  if constexpr (LT == 0) {
    if (gbase == nullptr) return;   // scores only (indexer_scores)
    const int64_t G = (N + kGroup - 1) / kGroup;
    float* grow = gbase + (r - grow0) * G;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int64_t e0 = batch_base(i);
      if (col == 0 && e0 + 16 * g < nvis) grow[(e0 + 16 * g) / kGroup] = out_g[i];
    }
  } else {
    static_assert(NB == 4 && LT <= 64, "list mode sorts four composites per lane");
    unsigned long long c[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int64_t e = batch_base(i) + lane;
      c[i] = e < nvis ? composite(order_key(out_s[i]), e) : 0ull;
    }
    auto cas = [](unsigned long long& a, unsigned long long& b) {   // a >= b afterwards
      const unsigned long long hi = a > b ? a : b, lo = a > b ? b : a;
      a = hi;
      b = lo;
    };
    cas(c[0], c[1]); cas(c[2], c[3]); cas(c[0], c[2]); cas(c[1], c[3]); cas(c[1], c[2]);
    unsigned long long mine = 0ull;
#pragma unroll
    for (int t = 0; t < LT; ++t) {
      const uint32_t hk = (uint32_t)(c[0] >> 32), hi = (uint32_t)c[0];
      const uint32_t mk = wave_max_u32(hk);
      const unsigned long long tied = __ballot(hk == mk);
      uint32_t mi;
      if (__popcll(tied) == 1) {   // wave-uniform; the usual case: one lane holds the key
        mi = __builtin_amdgcn_readlane(hi, __ffsll((long long)tied) - 1);
      } else {
        mi = wave_max_u32(hk == mk ? hi : 0u);
      }
      const unsigned long long top = ((unsigned long long)mk << 32) | mi;
      if (lane == t) mine = top;
      if (c[0] == top) {   // the lane that held it (all lanes once every composite is 0)
        c[0] = c[1];
        c[1] = c[2];
        c[2] = c[3];
        c[3] = 0ull;
      }
    }
    const int64_t X = gridDim.x;
    unsigned long long* lrow = lbase + (r - lrow0) * (4 * X * LT) + ((int64_t)blockIdx.x * 4 + wv) * LT;
    if (lane < LT) lrow[lane] = mine;
  }
}

// ------------------------------------------------------------------ prefill score kernel (fp8 / fp4)
// Quantised keys with d_I = 128, four consecutive queries of one sequence per
// block of four waves, one query per wave (so only that query's operands and
// weights stay in registers). The block streams its entry range through an
// LDS ring of kPfDepth stages of 64 entries (key rows plus one 32-bit scale
// word per entry: the fp8 row scale, or the four E8M0 block scales of an fp4
// row), filled by global_load_lds: wave w copies rows 16w .. 16w + 15 of each
// stage (fp8: two dwordx4 loads, fp4: one) and their scale words (one dword
// load, 16 lanes), so every wave has the same number of loads per stage in
// flight. Within a row, 16-byte chunk c is stored at position
// c ^ ((row >> 1) & 7) (fp8, 128-byte rows) or c ^ ((row >> 2) & 3) (fp4,
// 64-byte rows): the 16 rows read by the 16 lanes of one B-operand load then
// fall on 16 distinct bank groups.
//
// Each wave scores all 64 entries of a stage for its query: 4 tiles x HB
// head blocks of v_mfma_scale_f32_16x16x128_f8f6f4 (fp4: the E8M0 block
// scales of query and key go to the instruction's scale operands), the
// weighted ReLU head sum in registers and one reduce-scatter that leaves lane
// l with entry base + l. Its score row segment (one 256-byte store) and group
// maxima are stored one stage later, so a store is never the last memory
// operation before a wait: waits count only loads issued after the awaited
// stage, which also covers every earlier store (vmcnt counts both). Blocks run
// the longest rows (last query groups) first.
constexpr int kPfStage = 64;
constexpr int kPfDepth = 4;

template <int FMT> struct PfCfg;
template <> struct PfCfg<CSA_FP8_E4M3> {
  static constexpr int RB = 128;   // bytes per key row
  static constexpr int LOADS = 3;  // loads per stage per wave
};
template <> struct PfCfg<CSA_FP4_E2M1> {
  static constexpr int RB = 64;
  static constexpr int LOADS = 2;
};

template <int FMT, int HB, typename SC>
__global__ __launch_bounds__(256) void k_index_score_pf(
    const uint8_t* __restrict__ q_idx, const void* __restrict__ q_scale, const float* __restrict__ w,
    const uint8_t* __restrict__ k_idx, const void* __restrict__ k_scale, const int32_t* __restrict__ q_pos,
    int64_t Tq, int64_t N, int H_I, int ratio, int64_t group0, int64_t groups_per_batch,
    int64_t chunk_entries, SC* __restrict__ sbase, int64_t srow0, float* __restrict__ gbase, int64_t grow0) {
  constexpr bool F4 = FMT == CSA_FP4_E2M1;
  constexpr int RB = PfCfg<FMT>::RB, LOADS = PfCfg<FMT>::LOADS;
  constexpr int SB = kPfStage * RB;   // key bytes per stage
  __shared__ __align__(16) uint8_t ring[kPfDepth][SB];
  __shared__ __align__(16) uint32_t sring[kPfDepth][kPfStage];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int g = lane >> 4, col = lane & 15;
  const int64_t grp = group0 + (int64_t)(gridDim.y - 1 - blockIdx.y);
  const int64_t b = grp / groups_per_batch;
  const int64_t t0 = (grp % groups_per_batch) * 4;
  const int nq = (int)((Tq - t0) < 4 ? (Tq - t0) : 4);
  int64_t nmax = 0, nvw = 0;
#pragma unroll
  for (int qi = 0; qi < 4; ++qi) {
    const int64_t n = qi < nq ? visible(q_pos[b * Tq + t0 + qi], ratio, N) : 0;
    nmax = n > nmax ? n : nmax;
    nvw = qi == wv ? n : nvw;
  }
  const int64_t e_begin = (int64_t)blockIdx.x * chunk_entries;
  if (e_begin >= nmax) return;
  const int64_t e_end = (e_begin + chunk_entries) < nmax ? (e_begin + chunk_entries) : nmax;
  const int S = (int)((e_end - e_begin + kPfStage - 1) / kPfStage);
  const bool live_q = wv < nq;
  const int64_t r = b * Tq + t0 + (live_q ? wv : 0);

  // Query operands (A: head = lane % 16 of head block hb; fp8: K bytes
  // [32g, 32g + 32), fp4: K elements [32g, 32g + 32) = bytes [16g, 16g + 16)
  // with their E8M0 block scale) and weights (fp8: the query's row scale
  // folded in); padded heads are zero.
  i32x8 qa[HB];
  int qs8[HB];
  float wq[HB][4];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int hrow = hb * 16 + col;
    const bool live = hrow < H_I;
    const int64_t qr = r * H_I + (live ? hrow : 0);
    if constexpr (F4) {
      const i32x4 x0 = *reinterpret_cast<const i32x4*>(q_idx + qr * RB + 16 * g);
      qa[hb] = live ? i32x8{x0[0], x0[1], x0[2], x0[3], 0, 0, 0, 0} : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      const int sc = reinterpret_cast<const uint8_t*>(q_scale)[qr * 4 + g];
      qs8[hb] = live ? sc : 127;
    } else {
      const uint8_t* qrow = q_idx + qr * RB + 32 * g;
      const i32x4 x0 = *reinterpret_cast<const i32x4*>(qrow);
      const i32x4 x1 = *reinterpret_cast<const i32x4*>(qrow + 16);
      qa[hb] = live ? i32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]} : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      qs8[hb] = 127;
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int h = hb * 16 + 4 * g + rr;
      const int hs = h < H_I ? h : 0;
      float wv_ = w[r * H_I + hs];
      if constexpr (!F4) wv_ *= reinterpret_cast<const float*>(q_scale)[r * H_I + hs];
      wq[hb][rr] = h < H_I ? wv_ : 0.f;
    }
  }
  wait_vm<0>();   // the operand loads above are complete before the ring's loads start

  const uint8_t* kb = k_idx + b * N * RB;
  const uint32_t* ksb = reinterpret_cast<const uint32_t*>(k_scale) + b * N;
  const uint32_t ring0 = (uint32_t)(uintptr_t)&ring[0][0];
  const uint32_t sring0 = (uint32_t)(uintptr_t)&sring[0][0];
  // Stage loads: rows past N - 1 read row N - 1 (scores of entries past the
  // visible count are never stored). One dwordx4 load covers 1 KB: 8 rows
  // (fp8) or 16 rows (fp4).
  constexpr int RPL = 1024 / RB;                 // rows per load
  constexpr int CPR = RB / 16;                   // chunks per row
  const int rA = 16 * wv + lane / CPR;           // row of the first load (+8 for the second, fp8)
  auto swz = [](int row) { return F4 ? ((row >> 2) & 3) : ((row >> 1) & 7); };
  const uint32_t cA = (uint32_t)((lane % CPR) ^ swz(rA));
  const uint32_t cB = (uint32_t)((lane % CPR) ^ swz(rA + 8));
  auto issue = [&](int st) {
    const int64_t e0 = e_begin + (int64_t)kPfStage * st;
    const int64_t eb = e0 < N - 1 ? e0 : N - 1;                     // uniform
    const int lim = (int)((N - 1 - eb) < (kPfStage - 1) ? (N - 1 - eb) : (kPfStage - 1));
    const uint8_t* sb = kb + eb * RB;
    const uint32_t slot = ring0 + (uint32_t)(st % kPfDepth) * SB;
    const uint32_t ra = (uint32_t)(rA < lim ? rA : lim);
    gather_lds16_s(sb, ra * RB + 16u * cA, slot + (uint32_t)(16 * wv) * RB);
    if constexpr (!F4) {
      const uint32_t rb = (uint32_t)(rA + 8 < lim ? rA + 8 : lim);
      gather_lds16_s(sb, rb * RB + 16u * cB, slot + (uint32_t)(16 * wv + RPL) * RB);
    }
    if (lane < 16) {
      const int rs = 16 * wv + lane;
      gather_lds4_s(ksb + eb, 4u * (uint32_t)(rs < lim ? rs : lim),
                    sring0 + (uint32_t)(st % kPfDepth) * (kPfStage * 4) + (uint32_t)(64 * wv));
    }
  };
#pragma unroll
  for (int st = 0; st < kPfDepth - 1; ++st)
    if (st < S) issue(st);

  // B-operand LDS offsets of this lane (tile t adds 16 * RB * t): row col;
  // fp8: chunks 2g and 2g + 1, fp4: chunk g; swizzled as stored
  const uint32_t sw = (uint32_t)swz(col);
  const uint32_t ob0 = F4 ? (uint32_t)col * RB + 16u * ((uint32_t)g ^ sw)
                          : (uint32_t)col * RB + 16u * ((2u * g) ^ sw);
  const uint32_t ob1 = (uint32_t)col * RB + 16u * ((2u * g + 1u) ^ sw);
  const int64_t G = (N + kGroup - 1) / kGroup;
  SC* srow = sbase + (r - srow0) * N;
  float* grow = gbase + (r - grow0) * G;
  float prev_s = 0.f, prev_g = 0.f;
  int64_t prev_e = -1;
  auto store_prev = [&]() {
    if (live_q && prev_e >= 0) {
      if (prev_e + lane < nvw) ScoreT<SC>::store(srow, prev_e + lane, prev_s);
      if (gbase && col == 0 && prev_e + 16 * g < nvw) grow[(prev_e + 16 * g) / kGroup] = prev_g;
    }
  };
  for (int st = 0; st < S; ++st) {
    if (st + kPfDepth - 2 < S) wait_vm<(kPfDepth - 2) * LOADS>();
    else if (st + 1 < S) wait_vm<LOADS>();
    else wait_vm<0>();
    __syncthreads();   // stage st is in LDS; every wave is done with stage st - 1
    if (st + kPfDepth - 1 < S) issue(st + kPfDepth - 1);
    store_prev();
    if (live_q) {
      uint32_t kslot = ring0 + (uint32_t)(st % kPfDepth) * SB;
      opaque(kslot);
      uint32_t sslot = sring0 + (uint32_t)(st % kPfDepth) * (kPfStage * 4);
      float part[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        i32x8 bv;
        int ks8 = 127;
        if constexpr (F4) {
          const i32x4 b0 = lds_read_b128(kslot + ob0 + (uint32_t)(16 * RB * t));
          bv = i32x8{b0[0], b0[1], b0[2], b0[3], 0, 0, 0, 0};
          const uint32_t sw4 = *(__attribute__((address_space(3))) const uint32_t*)(size_t)(sslot + 4u * (16 * t + col));
          ks8 = (int)((sw4 >> (8 * g)) & 0xffu);
        } else {
          const i32x4 b0 = lds_read_b128(kslot + ob0 + (uint32_t)(16 * RB * t));
          const i32x4 b1 = lds_read_b128(kslot + ob1 + (uint32_t)(16 * RB * t));
          bv = i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        }
        float pt = 0.f;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          f32x4 acc;
          if constexpr (F4)
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[hb], bv, f32x4{0.f, 0.f, 0.f, 0.f}, 4, 4, 0,
                                                                   qs8[hb], 0, ks8);
          else
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[hb], bv, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                                   127, 0, 127);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) pt = fmaf(wq[hb][rr], relu_bits(acc[rr]), pt);
        }
        part[t] = pt;
      }
      float sc = reduce_scatter4(part[0], part[1], part[2], part[3]);
      if constexpr (!F4) sc *= __uint_as_float(sring[st % kPfDepth][lane]);
      sc = ScoreT<SC>::round(sc);
      const int64_t e0 = e_begin + (int64_t)kPfStage * st;
      prev_s = sc;
      if (gbase) prev_g = max_row16(e0 + lane < nvw ? sc : -INFINITY);   // uniform: only a selection that reads them
      prev_e = e0;
    }
  }
  store_prev();
}

// ------------------------------------------------------------------ block helpers

// Inclusive scan across the block of one value per thread (kTopkThreads
// threads); the wave sums are left in wsum[0 .. waves).
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  v = wave_incl_sum(v);
  if (lane == 63) wsum[wv] = v;
  __syncthreads();
  uint32_t add = 0;
  for (int i = 0; i < wv; ++i) add += wsum[i];
  __syncthreads();
  return v + add;
}

struct TopkSmem {
  uint32_t hist[kHistBins];
  unsigned long long cand[kCandCap];
  int sel[kMaxK];
  uint32_t h256[256];
  uint32_t wsum[16];
  unsigned long long red_and[kTopkThreads / 64], red_or[kTopkThreads / 64];
  float redf[kTopkThreads / 64], redg[kTopkThreads / 64];
  int nsel, ncand, ngrp;
  uint32_t bin, need;
  unsigned long long prefix, mask, thresh;
  int done;
};

// Bucket of the target-th largest element of sm.hist (bins scanned from the
// top); sets sm.bin and sm.need = target - (count in higher bins).
__device__ void find_bucket(TopkSmem& sm, uint32_t target) {
  const int tid = threadIdx.x;
  constexpr int BPT = kHistBins / kTopkThreads;
  const int top = kHistBins - BPT * tid;   // owns bins [top - BPT, top)
  uint32_t mine = 0;
#pragma unroll
  for (int i = 1; i <= BPT; ++i) mine += sm.hist[top - i];
  const uint32_t incl = block_inclusive_scan(mine, sm.wsum);
  const uint32_t excl = incl - mine;
  if (excl < target && incl >= target) {
    uint32_t above = excl;
    int bin = top - 1;
    for (; bin > top - BPT; --bin) {
      if (above + sm.hist[bin] >= target) break;
      above += sm.hist[bin];
    }
    sm.bin = (uint32_t)bin;
    sm.need = target - above;
  }
  __syncthreads();
}

// Radix select: the need-th largest composite among alive elements (those
// whose masked bits equal the prefix). get(i, ok) returns element i's key.
// First the bits on which every alive element agrees are fixed at once (AND /
// OR reduction); then 8-bit digits are resolved from the top, each with a
// 256-bin LDS histogram and a one-wave parallel search for the digit that
// holds the need-th largest. Stops as soon as the chosen digit's bucket is
// taken whole.
template <typename Get>
__device__ void radix_threshold(TopkSmem& sm, int64_t count, Get get) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  {
    unsigned long long a = ~0ull, o = 0ull;
    const unsigned long long mask = sm.mask, prefix = sm.prefix;
    for (int64_t i = tid; i < count; i += kTopkThreads) {
      bool ok;
      const unsigned long long key = get(i, ok);
      if (ok && (key & mask) == prefix) { a &= key; o |= key; }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      a &= __shfl_xor(a, off);
      o |= __shfl_xor(o, off);
    }
    if (lane == 0) { sm.red_and[wv] = a; sm.red_or[wv] = o; }
    __syncthreads();
    if (tid == 0) {
      unsigned long long A = ~0ull, Ov = 0ull;
      for (int w = 0; w < kTopkThreads / 64; ++w) { A &= sm.red_and[w]; Ov |= sm.red_or[w]; }
      const unsigned long long diff = A ^ Ov;          // bits on which alive keys differ
      const int lead = diff ? __clzll(diff) : 64;
      const unsigned long long lm = lead >= 64 ? ~0ull : (lead == 0 ? 0ull : (~0ull << (64 - lead)));
      if ((lm | sm.mask) != sm.mask) {
        sm.mask |= lm;
        sm.prefix = A & sm.mask;
      }
      sm.done = sm.mask == ~0ull;
      sm.thresh = sm.prefix;
    }
    __syncthreads();
    if (sm.done) return;
  }
  for (;;) {
    const int fixed = __popcll(sm.mask);
    const int width = (64 - fixed) < 8 ? (64 - fixed) : 8;
    const int shift = 64 - fixed - width;
    const unsigned long long dmask = ((1ull << width) - 1ull) << shift;
    for (int i = tid; i < 256; i += kTopkThreads) sm.h256[i] = 0;
    __syncthreads();
    const unsigned long long mask = sm.mask, prefix = sm.prefix;
    for (int64_t i = tid; i < count; i += kTopkThreads) {
      bool ok;
      const unsigned long long key = get(i, ok);
      if (ok && (key & mask) == prefix) atomicAdd(&sm.h256[(key & dmask) >> shift], 1u);
    }
    __syncthreads();
    if (wv == 0) {
      // lane l owns digits [252 - 4l, 255 - 4l], scanned from the top
      const int top = 255 - 4 * lane;
      uint32_t h[4], mine = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { h[j] = sm.h256[top - j]; mine += h[j]; }
      const uint32_t incl = wave_incl_sum(mine);
      const uint32_t need = sm.need, excl = incl - mine;
      if (excl < need && incl >= need) {
        uint32_t above = excl;
        int j = 0;
        for (; j < 3; ++j) {
          if (above + h[j] >= need) break;
          above += h[j];
        }
        const int dd = top - j;
        const uint32_t rest = need - above;
        sm.prefix = prefix | ((unsigned long long)dd << shift);
        sm.mask = mask | dmask;
        sm.need = rest;
        sm.done = (h[j] == rest) || (sm.mask == ~0ull);
        sm.thresh = sm.prefix;   // remaining low bits zero: key >= thresh <=> chosen
      }
    }
    __syncthreads();
    if (sm.done) break;
  }
}

// Append slot for each lane with pred set: one atomic per wave (ballot +
// prefix popcount). Returns -1 for lanes without pred.
__device__ __forceinline__ int wave_append(bool pred, int* counter) {
  const unsigned long long mask = __ballot(pred);
  if (mask == 0ull) return -1;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)mask) - 1;
  int base = 0;
  if (lane == leader) base = atomicAdd(counter, __popcll(mask));
  base = __shfl(base, leader);
  return pred ? base + __popcll(mask & ((1ull << lane) - 1ull)) : -1;
}

__device__ __forceinline__ float block_min(float v, float* red) {
  v = wave_min(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kTopkThreads / 64; ++w) r = fminf(r, red[w]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kTopkThreads / 64; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

// Write the keff distinct indices of sm.sel in ascending order. For rows of
// up to 32 * kHistBins entries a bitmap of the chosen entries is built in the
// (then unused) histogram area and compacted in order with one block scan;
// longer rows place each index at its rank among the chosen.
__device__ void write_sorted(TopkSmem& sm, int keff, int64_t n, int32_t* __restrict__ out) {
  const int tid = threadIdx.x;
  if (n <= (int64_t)32 * kHistBins) {
    constexpr int WPT = kHistBins / kTopkThreads;          // bitmap words per thread
    for (int i = tid; i < kHistBins; i += kTopkThreads) sm.hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < keff; i += kTopkThreads) {
      const int v = sm.sel[i];
      atomicOr(&sm.hist[v >> 5], 1u << (v & 31));
    }
    __syncthreads();
    uint32_t w[WPT], cnt = 0;
#pragma unroll
    for (int j = 0; j < WPT; ++j) { w[j] = sm.hist[tid * WPT + j]; cnt += __popc(w[j]); }
    const uint32_t incl = block_inclusive_scan(cnt, sm.wsum);
    int pos = (int)(incl - cnt);
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      uint32_t x = w[j];
      while (x) {
        const int bit = __ffs((int)x) - 1;
        out[pos++] = (tid * WPT + j) * 32 + bit;
        x &= x - 1u;
      }
    }
    return;
  }
  for (int i = tid; i < keff; i += kTopkThreads) {
    const int v = sm.sel[i];
    int rank = 0;
#pragma unroll 8
    for (int j = 0; j < keff; ++j) rank += sm.sel[j] < v;
    out[rank] = v;
  }
}

// Take the candidates whose composite is >= the need-th largest among
// sm.cand[0..ncand) into sm.sel (appending after sm.nsel).
__device__ void take_top_candidates(TopkSmem& sm, int ncand) {
  const int tid = threadIdx.x;
  if ((uint32_t)ncand == sm.need) {
    for (int c = tid; c < ncand; c += kTopkThreads) sm.sel[atomicAdd(&sm.nsel, 1)] = composite_index(sm.cand[c]);
  } else {
    radix_threshold(sm, ncand, [&](int64_t i, bool& ok) { ok = true; return sm.cand[i]; });
    const unsigned long long th = sm.thresh;
    for (int c = tid; c < ncand; c += kTopkThreads)
      if (sm.cand[c] >= th) sm.sel[atomicAdd(&sm.nsel, 1)] = composite_index(sm.cand[c]);
  }
  __syncthreads();
}

// Full-row path: 13-bit histogram of all n scores, take the higher buckets,
// resolve the boundary bucket exactly. Leaves k indices in sm.sel.
template <typename SC>
__device__ void select_full_row(TopkSmem& sm, const SC* __restrict__ srow, int64_t n, int k) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kHistBins; i += kTopkThreads) sm.hist[i] = 0;
  if (tid == 0) { sm.nsel = 0; sm.ncand = 0; }
  __syncthreads();
#pragma unroll 8
  for (int64_t i = tid; i < n; i += kTopkThreads)
    atomicAdd(&sm.hist[order_key(ScoreT<SC>::load(srow, i)) >> (32 - kHistBits)], 1u);
  __syncthreads();
  find_bucket(sm, (uint32_t)k);
  const uint32_t d1 = sm.bin;
#pragma unroll 8
  for (int64_t i = tid; i < n; i += kTopkThreads) {
    const uint32_t key = order_key(ScoreT<SC>::load(srow, i));
    const uint32_t d = key >> (32 - kHistBits);
    if (d > d1) {
      sm.sel[atomicAdd(&sm.nsel, 1)] = (int)i;
    } else if (d == d1) {
      const int c = atomicAdd(&sm.ncand, 1);
      if (c < kCandCap) sm.cand[c] = composite(key, i);
    }
  }
  __syncthreads();
  const int ncand = sm.ncand;
  if (tid == 0) {
    sm.prefix = (unsigned long long)d1 << (64 - kHistBits);
    sm.mask = ~0ull << (64 - kHistBits);
    sm.done = 0;
  }
  __syncthreads();
  if (ncand <= kCandCap) {
    take_top_candidates(sm, ncand);
  } else {
    // Bucket larger than the LDS list (heavy ties): select straight from the row.
    radix_threshold(sm, n, [&](int64_t i, bool& ok) {
      ok = true;
      return composite(order_key(ScoreT<SC>::load(srow, i)), i);
    });
    const unsigned long long th = sm.thresh;
    for (int64_t i = tid; i < n; i += kTopkThreads) {
      const uint32_t key = order_key(ScoreT<SC>::load(srow, i));
      if ((key >> (32 - kHistBits)) == d1 && composite(key, i) >= th) sm.sel[atomicAdd(&sm.nsel, 1)] = (int)i;
    }
    __syncthreads();
  }
}

// Group path (one row, kTopkThreads = 1024 threads).
//
// Let G_k be the k-th largest group maximum. The k largest maxima are k
// distinct entries >= G_k, so the k-th largest entry K* is >= G_k. The maxima
// are binned linearly between their minimum and maximum; the map is monotone,
// so with b the bin of G_k every entry of the top-k has bin >= b and lies in a
// group whose maximum has bin >= b. Those groups are listed in index order
// (one block scan); their entries with bin >= b are the candidates, again
// compacted in index order. A second linear histogram over the candidates'
// range finds the bin b2 that holds the k-th largest candidate; candidates in
// higher bins are taken, and the ones in bin b2 are ranked among themselves
// by (score descending, index ascending). The chosen candidates are still in
// index order, so one more block scan writes the output.
//
// Each thread holds 16 consecutive group maxima in registers; 4096-bin
// histograms; up to 4096 listed groups and 4096 candidates. Returns false
// (nothing written) when the row does not fit these bounds (heavy ties).
constexpr int kGPT = 16;                     // group maxima per thread
constexpr int kGBins = 4096;                 // bins per histogram
constexpr int kMaxGrp = 4096;                // listed groups
constexpr int kMaxCand = 4096;               // candidates (cand[0 .. 4096))

__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Exclusive scan of one value per thread; returns the exclusive prefix and
// the block total. One barrier: the caller must pass another barrier before
// wsum is written again.
__device__ __forceinline__ uint32_t block_scan_excl(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_sum(v);
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  uint32_t add = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kTopkThreads / 64; ++i) {
    const uint32_t x = wsum[i];
    add += i < wv ? x : 0u;
    tot += x;
  }
  total = tot;
  return add + incl - v;
}

// Boundary bin of the target-th largest element of hist[0 .. kGBins): sets
// sm.bin and sm.need (target minus the count in higher bins). Two barriers.
__device__ __forceinline__ void find_bin4096(TopkSmem& sm, const uint32_t* hist, uint32_t target) {
  constexpr int BPT = kGBins / kTopkThreads;
  const int top = kGBins - BPT * (int)threadIdx.x;    // owns bins [top - BPT, top)
  uint32_t h[BPT], mine = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) { h[i] = hist[top - 1 - i]; mine += h[i]; }
  uint32_t total;
  const uint32_t excl = block_scan_excl(mine, sm.wsum, total);
  if (excl < target && excl + mine >= target) {
    uint32_t above = excl;
    int i = 0;
    for (; i < BPT - 1; ++i) {
      if (above + h[i] >= target) break;
      above += h[i];
    }
    sm.bin = (uint32_t)(top - 1 - i);
    sm.need = target - above;
  }
  __syncthreads();
}

// a[j] for a register array a[0 .. 16) and a lane-varying j, as an OR of
// equality-masked bit patterns (a form that stays in registers; an indexed
// access would move the array to scratch memory).
__device__ __forceinline__ float pick16(const float (&a)[16], int j) {
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) r |= (uint32_t)(-(int32_t)(i == j)) & __float_as_uint(a[i]);
  return __uint_as_float(r);
}

template <typename SC>
__device__ bool select_by_groups(TopkSmem& sm, const SC* __restrict__ srow, const float* __restrict__ grow,
                                 int64_t n, int64_t m, int k, int32_t* __restrict__ out) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (m > (int64_t)kGPT * kTopkThreads) return false;
  uint32_t* hist1 = sm.hist;                    // group-maximum histogram, then the group list
  uint32_t* hist2 = sm.hist + kGBins;           // candidate histogram
  int* glist = reinterpret_cast<int*>(sm.hist);

  // 1. this thread's 16 consecutive group maxima (nv of them valid)
  float gv[kGPT];
  const int g0 = kGPT * tid;
  const int mi = (int)m, ni = (int)n;                    // m <= 16384, n < 2^30
  const int nv = mi - g0 < 0 ? 0 : (mi - g0 > kGPT ? kGPT : mi - g0);
  const bool vec_ok = (reinterpret_cast<uintptr_t>(grow) & 15) == 0;
  if (vec_ok && nv == kGPT) {
#pragma unroll
    for (int j = 0; j < kGPT; j += 4) {
      const float4 t4 = *reinterpret_cast<const float4*>(grow + g0 + j);
      gv[j] = t4.x; gv[j + 1] = t4.y; gv[j + 2] = t4.z; gv[j + 3] = t4.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kGPT; ++j) gv[j] = j < nv ? grow[g0 + j] : 0.f;
  }
  // 2. range of the maxima; clear both histograms meanwhile
#pragma unroll
  for (int i = tid; i < 2 * kGBins; i += kTopkThreads) sm.hist[i] = 0u;
  if (tid == 0) sm.nsel = 0;
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int j = 0; j < kGPT; ++j) {
    lo = j < nv ? fminf(lo, gv[j]) : lo;
    hi = j < nv ? fmaxf(hi, gv[j]) : hi;
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  if (lane == 0) { sm.redf[wv] = lo; sm.redg[wv] = hi; }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) { lo = fminf(lo, sm.redf[w]); hi = fmaxf(hi, sm.redg[w]); }
  const float inv = hi > lo ? (float)kGBins / (hi - lo) : 0.f;
  auto bin_of = [&](float v) -> int {
    const float t = (v - lo) * inv;
    return t >= (float)(kGBins - 1) ? kGBins - 1 : (int)t;    // monotone in v
  };
  // 3. histogram of the maxima (bins kept: -1 for invalid slots)
  int bn[kGPT];
#pragma unroll
  for (int j = 0; j < kGPT; ++j) {
    bn[j] = j < nv ? bin_of(gv[j]) : -1;
    if (j < nv) atomicAdd(&hist1[bn[j]], 1u);
  }
  __syncthreads();
  // 4. bin of the k-th largest maximum
  find_bin4096(sm, hist1, (uint32_t)k);
  const int b = (int)sm.bin;
  // 5. groups with bin >= b, listed in index order (hist1 is free now); tau,
  //    the smallest of their maxima, is <= G_k <= K*: entries >= tau are
  //    exactly the entries with bin >= b, a superset of the top-k
  uint32_t qual = 0;
  float tmin = INFINITY;
#pragma unroll
  for (int j = 0; j < kGPT; ++j) {
    const bool q = bn[j] >= b;
    qual |= (uint32_t)q << j;
    tmin = q ? fminf(tmin, gv[j]) : tmin;
  }
  tmin = wave_min(tmin);
  if (lane == 0) sm.redf[wv] = tmin;
  uint32_t ngrp;
  uint32_t pos = block_scan_excl((uint32_t)__popc(qual), sm.wsum, ngrp);   // its barrier also publishes redf
  if (ngrp > (uint32_t)kMaxGrp) return false;            // uniform
  float tau = INFINITY;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) tau = fminf(tau, sm.redf[w]);
  for (uint32_t qm = qual; qm; qm &= qm - 1u) glist[pos++] = g0 + __ffs((int)qm) - 1;
  __syncthreads();
  // 6. candidates: entries >= tau of the listed groups, in index order. Per
  //    round of up to 2048 groups every thread takes 0-2 consecutive ones.
  const bool svec = (reinterpret_cast<uintptr_t>(srow) & 15) == 0;
  uint32_t ncand = 0;
  for (uint32_t base = 0; base < ngrp; base += 2 * kTopkThreads) {
    const uint32_t cr = ngrp - base < 2u * kTopkThreads ? ngrp - base : 2u * kTopkThreads;
    const uint32_t ga = base + (uint32_t)tid * cr / kTopkThreads, gb = base + ((uint32_t)tid + 1) * cr / kTopkThreads;
    float va[kGroup], vb[kGroup];
    const int ea = ga < gb ? glist[ga] * kGroup : ni;
    const int eb = ga + 1 < gb ? glist[ga + 1] * kGroup : ni;
    if (svec && ea + kGroup <= ni) {
#pragma unroll
      for (int j = 0; j < kGroup; j += 8) load_scores8(srow + ea + j, va + j);
    } else {
#pragma unroll
      for (int j = 0; j < kGroup; ++j) va[j] = ea + j < ni ? ScoreT<SC>::load(srow, ea + j) : -INFINITY;
    }
    if (svec && eb + kGroup <= ni) {
#pragma unroll
      for (int j = 0; j < kGroup; j += 8) load_scores8(srow + eb + j, vb + j);
    } else {
#pragma unroll
      for (int j = 0; j < kGroup; ++j) vb[j] = eb + j < ni ? ScoreT<SC>::load(srow, eb + j) : -INFINITY;
    }
    uint32_t ma = 0, mb = 0;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {       // -inf past n fails
      ma |= (uint32_t)(va[j] >= tau) << j;
      mb |= (uint32_t)(vb[j] >= tau) << j;
    }
    uint32_t added;
    uint32_t p = ncand + block_scan_excl((uint32_t)(__popc(ma) + __popc(mb)), sm.wsum, added);
    for (uint32_t mk = ma; mk; mk &= mk - 1u) {
      const int j = __ffs((int)mk) - 1;
      if (p < (uint32_t)kMaxCand) sm.cand[p] = composite(order_key(pick16(va, j)), ea + j);
      ++p;
    }
    for (uint32_t mk = mb; mk; mk &= mk - 1u) {
      const int j = __ffs((int)mk) - 1;
      if (p < (uint32_t)kMaxCand) sm.cand[p] = composite(order_key(pick16(vb, j)), eb + j);
      ++p;
    }
    ncand += added;
    __syncthreads();
  }
  if (ncand > (uint32_t)kMaxCand) return false;          // uniform
  // 7. histogram of the candidates over [tau, hi]
  const float inv2 = hi > tau ? (float)kGBins / (hi - tau) : 0.f;
  auto bin2_of = [&](uint32_t key) -> int {
    const float t = (key_value(key) - tau) * inv2;
    return t >= (float)(kGBins - 1) ? kGBins - 1 : (int)t;
  };
  constexpr int CPT = kMaxCand / kTopkThreads;            // candidates per thread (consecutive)
  const uint32_t per = (ncand + kTopkThreads - 1) / kTopkThreads;
  unsigned long long cv[CPT];
  int cb[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const uint32_t ci = per * tid + j;
    const bool ok = j < (int)per && ci < ncand;
    cv[j] = ok ? sm.cand[ci] : 0ull;
    cb[j] = ok ? bin2_of((uint32_t)(cv[j] >> 32)) : -1;
    if (ok) atomicAdd(&hist2[cb[j]], 1u);
  }
  __syncthreads();
  find_bin4096(sm, hist2, (uint32_t)k);
  const int b2 = (int)sm.bin;
  const uint32_t need2 = sm.need;
  // 8. rank the candidates of bin b2 among themselves (list at cand[kMaxCand ..))
  unsigned long long* blist = sm.cand + kMaxCand;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int slot = wave_append(cb[j] == b2, &sm.nsel);
    if (slot >= 0) blist[slot] = cv[j];
  }
  __syncthreads();
  const int nb2 = sm.nsel;
  uint32_t take = 0, tcnt = 0;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    bool t = cb[j] > b2;
    if (cb[j] == b2) {
      if ((uint32_t)nb2 == need2) {
        t = true;
      } else {
        uint32_t rank = 0;
        for (int i = 0; i < nb2; ++i) rank += blist[i] > cv[j];
        t = rank < need2;
      }
    }
    take |= (uint32_t)t << j;
    tcnt += t;
  }
  // 9. write the chosen indices in ascending order
  uint32_t nout;
  uint32_t o = block_scan_excl(tcnt, sm.wsum, nout);
#pragma unroll
  for (int j = 0; j < CPT; ++j)
    if ((take >> j) & 1u) out[o++] = composite_index(cv[j]);
  return true;
}

// One block per row of the current pass. Row r's scores live at
// sbase + (r - srow0) * N and its group maxima at gbase + (r - grow0) * G.
template <typename SC>
__global__ __launch_bounds__(kTopkThreads) void k_topk_select(const SC* __restrict__ sbase, int64_t srow0,
                                                              const float* __restrict__ gbase, int64_t grow0,
                                                              int64_t row0, const int32_t* __restrict__ q_pos,
                                                              int64_t N, int ratio, int k, int32_t* __restrict__ idx_out) {
  __shared__ TopkSmem sm;
  const int tid = threadIdx.x;
  const int64_t r = row0 + blockIdx.x;
  const int64_t n = visible(q_pos[r], ratio, N);
  int32_t* out = idx_out + r * (int64_t)k;
  if (n <= k) {
    for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const int64_t G = (N + kGroup - 1) / kGroup;
  const SC* srow = sbase + (r - srow0) * N;
  const float* grow = gbase + (r - grow0) * G;
  const int64_t m = (n + kGroup - 1) / kGroup;
  if (m >= (int64_t)kGroupFactor * k && select_by_groups(sm, srow, grow, n, m, k, out)) return;
  __syncthreads();   // the group path may have been left part way: LDS is reused
  select_full_row(sm, srow, n, k);
  __syncthreads();
  write_sorted(sm, k, n, out);
}

// ------------------------------------------------------------------ list mode
// One block per row (kTopkThreads threads). The score kernel left, for each
// wave w of the row, the LT largest composites of the wave's entries, largest
// first (0 past the visible entries). Let C be the k-th largest composite of
// the union of the lists (exact: composites are distinct). If no wave's LT-th
// composite reaches C, then every entry >= C is listed (an unlisted entry of
// wave w is below w's LT-th composite, hence below C), so the listed
// composites >= C are exactly the row's top-k. Otherwise the waves whose
// LT-th composite is >= C ("full" waves) may hold more entries >= C: their
// unlisted entries >= C are read from the stored scores, and the top-k is
// selected exactly among the listed composites >= C and those entries (all
// entries >= C are among them, and there are at least k). Rows whose lists
// do not fit the kernel's bounds take the full-row path.
//
// C comes from a linear 4096-bin histogram of the composites' keys over
// [min, max] (a monotone map): composites in bins above the bin b of the k-th
// largest are chosen; those of bin b are compacted and each is ranked among
// them by one thread. The chosen entries are marked in a bitmap of the row
// (rows of at most 32 * 8192 entries) and written in ascending order after
// one block scan. Each phase costs a few barriers and at most one LDS round
// trip per wave (per-lane counts go through a wave prefix sum and one
// atomic per wave), because a block per row is latency-bound.
constexpr int kListPerThread = 16;
constexpr int kListCap = kListPerThread * kTopkThreads;   // composites per row
constexpr int kListFullWaves = 64;                        // full waves read back at most
constexpr int64_t kListMaxN = (int64_t)32 * kHistBins;    // entries covered by the bitmap

template <int LT, typename SC>
__global__ __launch_bounds__(kTopkThreads) void k_topk_lists(const SC* __restrict__ sbase, int64_t srow0,
                                                             const unsigned long long* __restrict__ lbase,
                                                             int64_t lrow0, int64_t X, int64_t row0,
                                                             const int32_t* __restrict__ q_pos, int64_t N, int ratio,
                                                             int k, int32_t* __restrict__ idx_out) {
  __shared__ TopkSmem sm;
  static_assert(kTopkThreads % LT == 0, "a wave's last slot sits in a fixed thread residue");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t r = row0 + blockIdx.x;
  const int64_t n = visible(q_pos[r], ratio, N);
  int32_t* out = idx_out + r * (int64_t)k;
  if (n <= k) {
    for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
    return;
  }
  const SC* srow = sbase + (r - srow0) * N;
  auto full_row = [&]() {   // uniform call sites, after a barrier
    select_full_row(sm, srow, n, k);
    __syncthreads();
    write_sorted(sm, k, n, out);
  };
  // lists of the score blocks that saw visible entries (block x's first
  // entry is 256 x)
  const int64_t xv = (n + 255) / 256 < X ? (n + 255) / 256 : X;
  const int64_t nl = xv * 4 * LT;
  if (nl > kListCap || n > kListMaxN) {   // uniform
    full_row();
    return;
  }
  const unsigned long long* lrow = lbase + (r - lrow0) * (4 * X * LT);
  // 1. composites: slot j * kTopkThreads + tid (coalesced loads). Slot sl is
  //    the (sl % LT)-th of wave sl / LT; this thread's slots all share the
  //    residue tid % LT.
  unsigned long long cv[kListPerThread];
#pragma unroll
  for (int j = 0; j < kListPerThread; ++j) {
    const int64_t sl = (int64_t)j * kTopkThreads + tid;
    cv[j] = sl < nl ? lrow[sl] : 0ull;
  }
  const bool last_slot = (tid % LT) == LT - 1;
  // 2. clear the histogram and the bitmap; key range and count of the nonzero
  //    composites (wave reductions, one LDS word each per wave)
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(sm.cand);   // kHistBins words, cand[0 .. kMaxCand)
  unsigned long long* blist = sm.cand + kMaxCand;             // composites of bin b
  for (int i = tid; i < kGBins; i += kTopkThreads) sm.hist[i] = 0u;
  for (int i = tid; i < kHistBins; i += kTopkThreads) bitmap[i] = 0u;
  if (tid == 0) { sm.nsel = 0; sm.ngrp = 0; sm.ncand = 0; sm.thresh = 1ull; }
  uint32_t kmin = 0xffffffffu, kmax = 0u, nzw = 0u;
#pragma unroll
  for (int j = 0; j < kListPerThread; ++j) {
    const uint32_t key = (uint32_t)(cv[j] >> 32);
    const bool nz = cv[j] != 0ull;
    if (nz) { kmin = min(kmin, key); kmax = max(kmax, key); }
    nzw += (uint32_t)__popcll(__ballot(nz));
  }
  kmax = wave_max_u32(kmax);
  kmin = ~wave_max_u32(~kmin);
  uint32_t* rmax = reinterpret_cast<uint32_t*>(sm.redg);
  uint32_t* rmin = reinterpret_cast<uint32_t*>(sm.redf);
  if (lane == 0) { rmax[wv] = kmax; rmin[wv] = kmin; sm.wsum[wv] = nzw; }
  __syncthreads();
  uint32_t total = 0;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) {
    kmax = max(kmax, rmax[w]);
    kmin = min(kmin, rmin[w]);
    total += sm.wsum[w];
  }
  const float inv = (float)kGBins / ((float)(kmax - kmin) + 1.f);
  auto bin_of = [&](uint32_t key) -> int {   // monotone in key
    const int t = (int)((float)(key - kmin) * inv);
    return t > kGBins - 1 ? kGBins - 1 : t;
  };
  // 3. histogram of the nonzero composites
  int bn[kListPerThread];
#pragma unroll
  for (int j = 0; j < kListPerThread; ++j) {
    bn[j] = cv[j] != 0ull ? bin_of((uint32_t)(cv[j] >> 32)) : -1;
    if (bn[j] >= 0) atomicAdd(&sm.hist[bn[j]], 1u);
  }
  __syncthreads();
  // With fewer than k listed composites, C stays 1: every listed one qualifies.
  if (total >= (uint32_t)k) {   // uniform
    // 4. bin b of the k-th largest composite
    find_bin4096(sm, sm.hist, (uint32_t)k);
    const int b = (int)sm.bin;
    const uint32_t need = sm.need;
    const uint32_t nb = sm.hist[b];
    if (nb > (uint32_t)(kCandCap - kMaxCand)) {   // uniform: a huge tie on one key range
      __syncthreads();
      full_row();
      return;
    }
    // 5. composites above bin b are chosen (marked now); those of bin b are
    //    compacted (a wave prefix sum of per-lane counts, one atomic per wave)
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < kListPerThread; ++j) {
      cnt += bn[j] == b;
      if (bn[j] > b) {
        const int e = composite_index(cv[j]);
        atomicOr(&bitmap[e >> 5], 1u << (e & 31));
      }
    }
    const uint32_t incl = wave_incl_sum(cnt);
    const uint32_t wtot = __builtin_amdgcn_readlane(incl, 63);
    uint32_t base = 0;
    if (wtot != 0) {   // uniform
      if (lane == 0) base = atomicAdd(reinterpret_cast<uint32_t*>(&sm.nsel), wtot);
      base = __builtin_amdgcn_readfirstlane(base);
    }
    uint32_t pos = base + incl - cnt;
#pragma unroll
    for (int j = 0; j < kListPerThread; ++j)
      if (bn[j] == b) blist[pos++] = cv[j];
    __syncthreads();
    // 6. rank of each bin-b composite among them (one thread each): C is the
    //    need-th largest; the need largest are chosen
    for (uint32_t e = tid; e < nb; e += kTopkThreads) {
      const unsigned long long c = blist[e];
      uint32_t rank = 0;
#pragma unroll 8
      for (uint32_t i = 0; i < nb; ++i) rank += blist[i] > c;
      if (rank == need - 1) sm.thresh = c;   // exactly one composite has this rank
      if (rank < need) {
        const int ei = composite_index(c);
        atomicOr(&bitmap[ei >> 5], 1u << (ei & 31));
      }
    }
    __syncthreads();
  }
  // 7. full waves: those whose last slot (LT-th composite) is >= C
  const unsigned long long C = sm.thresh;
  {
    uint32_t nf = 0;
#pragma unroll
    for (int j = 0; j < kListPerThread; ++j) nf += (uint32_t)__popcll(__ballot(last_slot && cv[j] != 0ull && cv[j] >= C));
    if (lane == 0 && nf != 0) atomicAdd(&sm.ngrp, (int)nf);
  }
  __syncthreads();
  const int nfull = sm.ngrp;
  // (nfull == 0 implies total >= k: with C = 1 a wave without a full list has
  // every visible entry listed, so no full wave would mean total = n > k)
  if (nfull == 0 && total >= (uint32_t)k) {   // uniform: exactly k composites are marked
    // 8. the chosen entries in ascending order: each thread counts the bits of
    //    its kHistBins / kTopkThreads bitmap words, one block scan places them
    constexpr int WPT = kHistBins / kTopkThreads;
    uint32_t wd[WPT], c = 0;
#pragma unroll
    for (int j = 0; j < WPT; ++j) { wd[j] = bitmap[tid * WPT + j]; c += __popc(wd[j]); }
    uint32_t tot;
    uint32_t o = block_scan_excl(c, sm.wsum, tot);
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      uint32_t x = wd[j];
      while (x) {
        const int bit = __ffs((int)x) - 1;
        out[o++] = (tid * WPT + j) * 32 + bit;
        x &= x - 1u;
      }
    }
    return;
  }
  if (nfull > kListFullWaves) {   // uniform: many full waves (ties, ordered scores)
    full_row();
    return;
  }
  // 9. (rare) the full waves, by their id sl / LT
  int* full = reinterpret_cast<int*>(sm.sel);
  __syncthreads();   // every thread has read nfull
  if (tid == 0) sm.ngrp = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kListPerThread; ++j) {
    const int64_t sl = (int64_t)j * kTopkThreads + tid;
    const int slot = wave_append(last_slot && cv[j] != 0ull && cv[j] >= C, &sm.ngrp);
    if (slot >= 0) full[slot] = (int)(sl / LT);
  }
  // 10. candidates: the listed composites >= C, then the unlisted entries >= C
  //     of the full waves (entries 64 (w' + 4 (x + X i)) + lane, i < 4, of
  //     wave 4 x + w'); the order of discovery does not matter below
#pragma unroll
  for (int j = 0; j < kListPerThread; ++j) {
    const int slot = wave_append(cv[j] != 0ull && cv[j] >= C, &sm.ncand);
    if (slot >= 0 && slot < kCandCap) sm.cand[slot] = cv[j];
  }
  __syncthreads();
  for (int f = wv; f < nfull; f += kTopkThreads / 64) {   // one full wave per wave of the block
    const int wid = full[f];
    const int64_t x = wid / 4, wq = wid % 4;
    const unsigned long long floor_c = lrow[(int64_t)wid * LT + LT - 1];   // its LT-th composite
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t e = 64 * (wq + 4 * (x + X * i)) + lane;
      unsigned long long c = 0ull;
      if (e < n) c = composite(order_key(ScoreT<SC>::load(srow, e)), e);
      const int slot = wave_append(c != 0ull && c >= C && c < floor_c, &sm.ncand);
      if (slot >= 0 && slot < kCandCap) sm.cand[slot] = c;
    }
  }
  __syncthreads();
  const int ncand = sm.ncand;
  __syncthreads();
  if (ncand > kCandCap) {   // uniform
    full_row();
    return;
  }
  // 11. exact top-k among the candidates (at least k: every entry >= C is one)
  if (tid == 0) {
    sm.nsel = 0;
    sm.prefix = 0ull;
    sm.mask = 0ull;
    sm.need = (uint32_t)k;
    sm.done = 0;
  }
  __syncthreads();
  take_top_candidates(sm, ncand);
  write_sorted(sm, k, n, out);
}

// ------------------------------------------------------------------ short rows
// Rows of n <= kSmallN scores (used for a whole launch when N <= kSmallN, e.g.
// prefill rows over the compressed entries of a 64k-token sequence): one
// 256-thread block per row; thread t keeps the order keys of entries
// [64 t, 64 t + 64) in registers, so the row is read once. Keys are taken
// relative to the row's smallest key (u = key - min, same order), and a 13-bit
// histogram covers the top 13 significant bits of the row's span, so a row
// whose scores lie close together still spreads over the bins (few
// same-address LDS atomics). The histogram gives the bucket d1 of the k-th
// largest key. Usual case (at most kSmallList keys in d1): one sweep marks the
// keys above d1 in a per-thread 64-bit mask and lists the keys of d1 as
// (u, inverted index) composites; a list key is chosen iff fewer than need of
// the list's composites exceed it. Otherwise a second histogram over the next
// 13 bits of the keys in d1 narrows the bucket, whose keys are ranked as
// composites (at most kSmallCand) or, for heavy ties, bisected over the
// remaining low bits of u (at most 6) and the inverted index. The chosen
// entries form a bitmap (one 64-bit word per thread); one block scan places
// them, staged in LDS and written out in order: ascending indices. Same total
// order (score descending, index ascending) as the general kernel.
constexpr int kSmallThreads = 256;
constexpr int kSmallPer = 64;
constexpr int64_t kSmallN = (int64_t)kSmallThreads * kSmallPer;   // 16384
constexpr int kSmallBits = 13;
constexpr int kSmallBins = 1 << kSmallBits;
constexpr int kSmallCand = 512;
constexpr int kSmallList = 256;

struct SmallSmem {
  uint32_t hist[kSmallBins + 64];   // + one spare bin per lane for entries past the row's end
  unsigned long long cand[kSmallCand];
  unsigned long long bits[kSmallThreads];   // chosen entries: bit j of word t is entry 64 t + j
  uint32_t wsum[kSmallThreads / 64];
  uint32_t wmin[kSmallThreads / 64], wmax[kSmallThreads / 64];
  uint32_t bin, need, ncand;
  unsigned long long thresh;
};

// Block-wide exclusive prefix of v (thread order) and total; one barrier.
__device__ __forceinline__ uint32_t small_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_sum(v);
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  uint32_t add = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kSmallThreads / 64; ++i) {
    const uint32_t x = wsum[i];
    add += i < wv ? x : 0u;
    tot += x;
  }
  total = tot;
  return add + incl - v;
}

__device__ __forceinline__ void small_clear(SmallSmem& sm) {
  uint4* h = reinterpret_cast<uint4*>(sm.hist);
#pragma unroll
  for (int i = 0; i < kSmallBins / 4 / kSmallThreads; ++i) h[threadIdx.x + i * kSmallThreads] = make_uint4(0u, 0u, 0u, 0u);
}

// Bucket of the target-th largest element of sm.hist (bins scanned from the
// top): sets sm.bin and sm.need (target minus the count in higher bins).
// Thread t sums bins [top - 32, top), top = kSmallBins - 32 t.
__device__ __forceinline__ void small_find(SmallSmem& sm, uint32_t target) {
  constexpr int BPT = kSmallBins / kSmallThreads;   // 32 bins per thread
  constexpr int G = BPT / 4;                        // groups of 4 bins
  const int top = kSmallBins - BPT * (int)threadIdx.x;
  const uint4* h = reinterpret_cast<const uint4*>(sm.hist + top - BPT);
  uint32_t gs[G], mine = 0;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const uint4 v = h[i];
    gs[i] = (v.x + v.y) + (v.z + v.w);
    mine += gs[i];
  }
  uint32_t total;
  const uint32_t excl = small_scan(mine, sm.wsum, total);
  if (excl < target && excl + mine >= target) {
    // the group (from the top) that holds the target, then the bin in it
    uint32_t above = excl;
    int gi = 0;
    bool done = false;
#pragma unroll
    for (int i = G - 1; i >= 0; --i) {
      const bool hit = !done && above + gs[i] >= target;
      gi = hit ? i : gi;
      done = done || hit;
      above += done ? 0u : gs[i];
    }
    const uint4 v = h[gi];
    const uint32_t c[4] = {v.w, v.z, v.y, v.x};
    uint32_t bin = 0, nd = 0;
    done = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool hit = !done && above + c[q] >= target;
      bin = hit ? (uint32_t)(top - BPT + 4 * gi + 3 - q) : bin;
      nd = hit ? target - above : nd;
      done = done || hit;
      above += c[q];
    }
    sm.bin = bin;
    sm.need = nd;
  }
  __syncthreads();
}

// The value passes through an empty asm statement: the compiler cannot reuse
// per-entry masks derived from it across passes (which would hold 64 lane
// masks in scalar registers and spill them).
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Pins a mask built bit by bit: the OR chain stays sequential (a balanced OR
// tree would hold all 64 bits in registers at once).
__device__ __forceinline__ void pin_mask(unsigned long long& t) {
  uint32_t lo = (uint32_t)t, hi = (uint32_t)(t >> 32);
  asm volatile("" : "+v"(lo), "+v"(hi));
  t = ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// Selection key of entry i (< kSmallN) with score v. float32 scores: the
// order key itself (ties are resolved later by index). bf16 scores carry only
// the high 16 bits of the order key, so the low 16 bits take 16383 - i: every
// key is distinct and orders entries by (score descending, index ascending),
// and equal bf16 scores, which are common, no longer pile into one histogram
// bin (same-address LDS atomics serialise).
template <typename SC>
__device__ __forceinline__ uint32_t small_key(float v, int i) {
  if constexpr (sizeof(SC) == 2)
    return (order_key(v) & 0xffff0000u) | (uint32_t)(kSmallN - 1 - i);
  else
    return order_key(v);
}

template <typename SC>
__global__ __launch_bounds__(kSmallThreads) void k_topk_small(const SC* __restrict__ sbase, int64_t srow0,
                                                              int64_t row0, const int32_t* __restrict__ q_pos,
                                                              int64_t N, int ratio, int k,
                                                              int32_t* __restrict__ idx_out) {
  __shared__ SmallSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t r = row0 + blockIdx.x;
  const int n = (int)visible(q_pos[r], ratio, N);   // <= kSmallN
  int32_t* out = idx_out + r * (int64_t)k;
  if (n <= k) {
    for (int i = tid; i < k; i += kSmallThreads) out[i] = i < n ? i : -1;
    return;
  }
  const SC* srow = sbase + (r - srow0) * N;
  const int base = tid * kSmallPer;
  const int nv = n - base < 0 ? 0 : (n - base > kSmallPer ? kSmallPer : n - base);
  uint32_t key[kSmallPer];
  uint32_t tmax = 0u, tinv = 0u;   // largest key and largest ~key (= ~smallest key) of the thread
  if (nv == kSmallPer && (reinterpret_cast<uintptr_t>(srow + base) & 15) == 0) {
#pragma unroll
    for (int j = 0; j < kSmallPer; j += 8) {
      float v[8];
      load_scores8(srow + base + j, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) key[j + i] = small_key<SC>(v[i], base + j + i);
    }
#pragma unroll
    for (int j = 0; j < kSmallPer; ++j) { tmax = max(tmax, key[j]); tinv = max(tinv, ~key[j]); }
  } else if (nv > 0) {
    // entries past the row's end repeat its last entry: the range is unchanged
    // and every later pass skips them (j >= nv)
#pragma unroll
    for (int j = 0; j < kSmallPer; ++j) {
      const int i = base + min(j, nv - 1);
      key[j] = small_key<SC>(ScoreT<SC>::load(srow, i), i);
    }
#pragma unroll
    for (int j = 0; j < kSmallPer; ++j) { tmax = max(tmax, key[j]); tinv = max(tinv, ~key[j]); }
  } else {
#pragma unroll
    for (int j = 0; j < kSmallPer; ++j) key[j] = 0u;
  }
  small_clear(sm);
  tmax = wave_umax(tmax);
  tinv = wave_umax(tinv);
  if (lane == 0) { sm.wmax[wv] = tmax; sm.wmin[wv] = tinv; }
  if (tid == 0) sm.ncand = 0u;
  __syncthreads();
  uint32_t kmax = 0u, kinv = 0u;
#pragma unroll
  for (int i = 0; i < kSmallThreads / 64; ++i) { kmax = max(kmax, sm.wmax[i]); kinv = max(kinv, sm.wmin[i]); }
  const uint32_t kmin = ~kinv;
#pragma unroll
  for (int j = 0; j < kSmallPer; ++j) key[j] -= kmin;   // u = key - kmin (order kept for the valid keys)
  const uint32_t span = kmax - kmin;
  const int bits = span ? 32 - __clz(span) : 0;
  const int s1 = bits > kSmallBits ? bits - kSmallBits : 0;   // u >> s1 < kSmallBins
  const int s2 = s1 > kSmallBits ? s1 - kSmallBits : 0;       // <= 6
  const int w2 = s1 - s2;                                     // bits of the second histogram in use
  // Each pass below takes its own copies of the loop-invariant values
  // (fresh), so no per-entry mask or shifted key is kept from one pass to the
  // next.
  const unsigned long long valid = nv >= kSmallPer ? ~0ull : ((1ull << nv) - 1ull);
  if (nv > 0) {  // pass 1
    const int nvp = fresh(nv), sp = fresh(s1);
#pragma unroll
    for (int j = 0; j < kSmallPer; ++j) atomicAdd(&sm.hist[j < nvp ? key[j] >> sp : kSmallBins + lane], 1u);
  }
  __syncthreads();
  small_find(sm, (uint32_t)k);
  const uint32_t d1 = sm.bin, need1 = sm.need;
  const uint32_t cnt1 = sm.hist[d1];
  unsigned long long take = 0;   // bit j: entry base + j is chosen
  if (cnt1 <= (uint32_t)kSmallList) {
    if (nv > 0) {
      const int nvp = fresh(nv), sp = fresh(s1);
#pragma unroll
      for (int j = 0; j < kSmallPer; ++j) {
        const uint32_t bj = key[j] >> sp;
        take |= (unsigned long long)(bj > d1) << j;
        if (j < nvp && bj == d1) sm.cand[atomicAdd(&sm.ncand, 1u)] = composite(key[j], base + j);
        if ((j & 7) == 7) pin_mask(take);
      }
    }
    sm.bits[tid] = take & valid;
    __syncthreads();
    if ((uint32_t)tid < cnt1) {
      const unsigned long long v = sm.cand[tid];
      uint32_t rank = 0;
      for (uint32_t e = 0; e < cnt1; ++e) rank += sm.cand[e] > v ? 1u : 0u;
      if (rank < need1) {
        const int i = composite_index(v);
        atomicOr(&sm.bits[i >> 6], 1ull << (i & 63));
      }
    }
    __syncthreads();
    take = sm.bits[tid];
  } else {
    small_clear(sm);
    __syncthreads();
    {  // pass 2: the next bits of the keys of bucket d1
      const int nvp = fresh(nv), sp = fresh(s1), sq = fresh(s2);
#pragma unroll
      for (int j = 0; j < kSmallPer; ++j)
        if (j < nvp && (key[j] >> sp) == d1) atomicAdd(&sm.hist[(key[j] >> sq) & (kSmallBins - 1)], 1u);
    }
    __syncthreads();
    small_find(sm, need1);
    // bucket pre of u >> s2; need >= 1 of its keys are taken
    const uint32_t pre = (d1 << w2) | (sm.bin & ((1u << w2) - 1u)), need = sm.need;
    uint32_t ceq = 0;
    {
      const int nvp = fresh(nv), sq = fresh(s2);
#pragma unroll
      for (int j = 0; j < kSmallPer; ++j) ceq += (j < nvp && (key[j] >> sq) == pre) ? 1u : 0u;
    }
    uint32_t ncand;
    uint32_t pos = small_scan(ceq, sm.wsum, ncand);
    uint32_t thu, thi;   // threshold (u, index): taken iff u > thu, or u == thu and index <= thi
    if (ncand <= (uint32_t)kSmallCand) {
      if (ceq) {
        const int nvp = fresh(nv), sq = fresh(s2);
#pragma unroll
        for (int j = 0; j < kSmallPer; ++j)
          if (j < nvp && (key[j] >> sq) == pre) sm.cand[pos++] = composite(key[j], base + j);
      }
      __syncthreads();
      for (uint32_t c = tid; c < ncand; c += kSmallThreads) {
        const unsigned long long v = sm.cand[c];
        uint32_t rank = 0;
        for (uint32_t e = 0; e < ncand; ++e) rank += sm.cand[e] > v ? 1u : 0u;
        if (rank == need - 1) sm.thresh = v;   // composites are distinct: exactly one
      }
      __syncthreads();
      thu = (uint32_t)(sm.thresh >> 32);
      thi = 0xffffffffu - (uint32_t)sm.thresh;
    } else {
      // Heavy ties: bisection over x = (low s2 bits of u, 16383 - index), which
      // orders the bucket's keys like their composites.
      uint32_t t = 0;
      for (int bt = s2 + 13; bt >= 0; --bt) {
        const uint32_t c = t | (1u << bt);
        const int nvp = fresh(nv), sq = fresh(s2);
        const uint32_t lowm = (1u << sq) - 1u;
        uint32_t cnt = 0;
#pragma unroll
        for (int j = 0; j < kSmallPer; ++j) {
          const uint32_t x = ((key[j] & lowm) << 14) | (uint32_t)(kSmallN - 1 - (base + j));
          cnt += (j < nvp && (key[j] >> sq) == pre && x >= c) ? 1u : 0u;
        }
        uint32_t tot;
        (void)small_scan(cnt, sm.wsum, tot);
        __syncthreads();   // wsum is rewritten by the next round
        if (tot >= need) t = c;
      }
      thu = (pre << s2) | (t >> 14);
      thi = (uint32_t)(kSmallN - 1) - (t & (uint32_t)(kSmallN - 1));
    }
    // taken: keys above the threshold key, and ties of it up to its index
    // (every key above bucket pre is above thu, which lies in the bucket)
#pragma unroll
    for (int j = 0; j < kSmallPer; ++j) {
      take |= (unsigned long long)(key[j] > thu || (key[j] == thu && (uint32_t)(base + j) <= thi)) << j;
      if ((j & 7) == 7) pin_mask(take);
    }
    take &= valid;
  }
  // Output: the chosen entries in index order (exactly k of them).
  uint32_t total;
  uint32_t o = small_scan((uint32_t)__popcll(take), sm.wsum, total);
  if (k <= kSmallBins) {
    uint32_t* stage = sm.hist;   // free once every thread has passed the scan
    while (take) {
      const int j = __builtin_ctzll(take);
      stage[o++] = (uint32_t)(base + j);
      take &= take - 1;
    }
    __syncthreads();
    if ((k & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
      for (int i = 4 * tid; i < k; i += 4 * kSmallThreads)
        *reinterpret_cast<uint4*>(out + i) = *reinterpret_cast<const uint4*>(stage + i);
    } else {
      for (int i = tid; i < k; i += kSmallThreads) out[i] = (int32_t)stage[i];
    }
  } else {
    while (take) {
      const int j = __builtin_ctzll(take);
      out[o++] = base + j;
      take &= take - 1;
    }
  }
}

// ------------------------------------------------------------------ host side

struct IndexPlan {
  int QB;
  int64_t groups_per_batch, groups, chunk_entries, groups_per_pass, max_rows_per_pass;
  bool dec;          // one query per block row: k_index_score_dec
  int lt;            // list mode (k_topk_lists): composites kept per wave, 0 = group maxima
  int64_t dec_x;     // decode grid width (blocks of 256 * kDecNB entries per row)
};

constexpr int kDecNB = 4, kDecDepth = 2;   // decode score kernel: batches per wave, ring depth

static IndexPlan make_plan(int64_t B, int64_t Tq, int64_t N, int sbytes, int d_I, csa_dtype fmt, int k) {
  IndexPlan p;
  p.QB = Tq >= 4 ? 4 : 1;
  p.groups_per_batch = cdiv(Tq, p.QB);
  p.groups = B * p.groups_per_batch;
  p.dec = p.QB == 1 && d_I == 128 && (fmt == CSA_FP8_E4M3 || fmt == CSA_FP4_E2M1);
  p.dec_x = cdiv(N > 0 ? N : 1, (int64_t)256 * kDecNB);
  // List mode for long decode rows: each wave of 256 entries keeps its LT
  // largest composites. About lambda = 256 k / N of a row's top-k fall in one
  // wave; LT covers lambda with a margin that leaves a wave full (more than
  // LT of its entries in the top-k, read back from the scores) rarely: LT 8
  // for lambda <= 1.25, 16 for lambda <= 5.
  p.lt = 0;
  if (p.dec && N > kSmallN) {
    const int lt = (int64_t)1024 * k <= 5 * N ? 8 : ((int64_t)256 * k <= 5 * N ? 16 : 0);
    if (lt > 0 && 4 * p.dec_x * lt <= kListCap && N <= kListMaxN) p.lt = lt;
  }
  // Score buffer budget per pass: 1 GiB.
  const int64_t budget = (int64_t)1 << 30;
  const int64_t row_bytes = (N > 0 ? N : 1) * sbytes + ((N + kGroup - 1) / kGroup) * 4 + 4 * p.dec_x * p.lt * 8;
  int64_t gpp = budget / (row_bytes * p.QB);
  if (gpp < 1) gpp = 1;
  if (gpp > 65535) gpp = 65535;
  if (gpp > p.groups) gpp = p.groups;
  p.groups_per_pass = gpp;
  p.max_rows_per_pass = gpp * p.QB;
  // Enough blocks per pass to cover the chip several times: split the
  // entries when a pass has few query groups.
  const int64_t want_blocks = 2048;
  int64_t chunks = cdiv(want_blocks, gpp);
  const int64_t max_chunks = cdiv(N, 256);
  if (chunks > max_chunks) chunks = max_chunks;
  if (chunks < 1) chunks = 1;
  p.chunk_entries = cdiv(cdiv(N, chunks), 64) * 64;
  if (p.chunk_entries < 64) p.chunk_entries = 64;
  return p;
}

static int64_t groups_of(int64_t N) { return (N + kGroup - 1) / kGroup; }

// Workspace: per pass, the scores [rows, N] (sbytes each: 4 for float32, 2 for
// bf16); from the next 256-byte boundary the group maxima [rows, G]; then,
// from the next 256-byte boundary, the list-mode composites [rows, 4 X LT].
static size_t score_area(const IndexPlan& p, int64_t N, int sbytes) {
  return ((size_t)p.max_rows_per_pass * (size_t)N * (size_t)sbytes + 255) / 256 * 256;
}
static size_t group_area(const IndexPlan& p, int64_t N) {
  return ((size_t)p.max_rows_per_pass * (size_t)groups_of(N) * 4 + 255) / 256 * 256;
}
size_t indexer_ws_bytes(int64_t B, int64_t Tq, int64_t N, int sbytes, int d_I, csa_dtype fmt, int k) {
  const IndexPlan p = make_plan(B, Tq, N, sbytes, d_I, fmt, k);
  const size_t lists = (size_t)p.max_rows_per_pass * (size_t)(4 * p.dec_x * p.lt) * 8;
  return score_area(p, N, sbytes) + group_area(p, N) + lists + 256;
}

// Batch shape of the key stream per format and queries per block (from
// sweeps on MI355X at the 262k/1M-context decode shapes and at the 65536-token
// and 8192-query prefill shapes: deeper batching or double buffering lowered
// occupancy without raising bandwidth, except 2 batches with 4 queries).
template <int FMT, int QB> struct ScoreCfg {
  static constexpr int UB = QB > 1 ? 2 : ((FMT == CSA_FP4_E2M1) ? 1 : 4);
  static constexpr bool DBUF = false;
};

// Decode score kernel shape (kDecNB, kDecDepth above): 4 batches of 64
// entries per wave, 2-deep ring (sweep at the 1M-context fp4 and 262k-context
// fp8 decode shapes).

template <int FMT, int LT, typename SC>
static void launch_score_dec_lt(int HB, dim3 grid, hipStream_t s, const void* q, const void* qs, const float* w,
                                const void* kk, const void* ks, const int32_t* qp, int64_t Tq, int64_t N, int H_I,
                                int ratio, int64_t r0, SC* sb, int64_t sr0, float* gb, int64_t gr0,
                                unsigned long long* lb, int64_t lr0) {
  switch (HB) {
    case 1: k_index_score_dec<FMT, 1, kDecNB, kDecDepth, LT, SC><<<grid, 256, 0, s>>>(q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, r0, sb, sr0, gb, gr0, lb, lr0); break;
    case 2: k_index_score_dec<FMT, 2, kDecNB, kDecDepth, LT, SC><<<grid, 256, 0, s>>>(q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, r0, sb, sr0, gb, gr0, lb, lr0); break;
    case 3: k_index_score_dec<FMT, 3, kDecNB, kDecDepth, LT, SC><<<grid, 256, 0, s>>>(q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, r0, sb, sr0, gb, gr0, lb, lr0); break;
    default: k_index_score_dec<FMT, 4, kDecNB, kDecDepth, LT, SC><<<grid, 256, 0, s>>>(q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, r0, sb, sr0, gb, gr0, lb, lr0); break;
  }
}

template <int FMT, typename SC>
static void launch_score_dec(int LT, int HB, dim3 grid, hipStream_t s, const void* q, const void* qs, const float* w,
                             const void* kk, const void* ks, const int32_t* qp, int64_t Tq, int64_t N, int H_I,
                             int ratio, int64_t r0, SC* sb, int64_t sr0, float* gb, int64_t gr0,
                             unsigned long long* lb, int64_t lr0) {
  if (LT == 8) launch_score_dec_lt<FMT, 8, SC>(HB, grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, r0, sb, sr0, gb, gr0, lb, lr0);
  else if (LT == 16) launch_score_dec_lt<FMT, 16, SC>(HB, grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, r0, sb, sr0, gb, gr0, lb, lr0);
  else launch_score_dec_lt<FMT, 0, SC>(HB, grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, r0, sb, sr0, gb, gr0, lb, lr0);
}

template <int FMT, int DI, int HB, int QB, typename SC>
static void launch_score(dim3 grid, hipStream_t s, const void* q, const void* qs, const float* w, const void* kk,
                         const void* ks, const int32_t* qp, int64_t Tq, int64_t N, int H_I, int ratio, int64_t g0,
                         int64_t gpb, int64_t ce, SC* sb, int64_t sr0, float* gb, int64_t gr0) {
  k_index_score<FMT, DI, HB, QB, ScoreCfg<FMT, QB>::UB, ScoreCfg<FMT, QB>::DBUF, SC><<<grid, 256, 0, s>>>(q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0, gb, gr0);
}

template <int FMT, int DI, int QB, typename SC>
static void dispatch_hb(int HB, dim3 grid, hipStream_t s, const void* q, const void* qs, const float* w,
                        const void* kk, const void* ks, const int32_t* qp, int64_t Tq, int64_t N, int H_I,
                        int ratio, int64_t g0, int64_t gpb, int64_t ce, SC* sb, int64_t sr0, float* gb, int64_t gr0) {
  switch (HB) {
    case 1: launch_score<FMT, DI, 1, QB, SC>(grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0, gb, gr0); break;
    case 2: launch_score<FMT, DI, 2, QB, SC>(grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0, gb, gr0); break;
    case 3: launch_score<FMT, DI, 3, QB, SC>(grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0, gb, gr0); break;
    default: launch_score<FMT, DI, 4, QB, SC>(grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0, gb, gr0); break;
  }
}

template <int FMT, typename SC>
static void launch_score_pf(int HB, dim3 grid, hipStream_t s, const void* q, const void* qs, const float* w,
                            const void* kk, const void* ks, const int32_t* qp, int64_t Tq, int64_t N, int H_I,
                            int ratio, int64_t g0, int64_t gpb, int64_t ce, SC* sb, int64_t sr0, float* gb,
                            int64_t gr0) {
  const auto* q8 = static_cast<const uint8_t*>(q);
  const auto* k8 = static_cast<const uint8_t*>(kk);
  switch (HB) {
    case 1: k_index_score_pf<FMT, 1, SC><<<grid, 256, 0, s>>>(q8, qs, w, k8, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0, gb, gr0); break;
    case 2: k_index_score_pf<FMT, 2, SC><<<grid, 256, 0, s>>>(q8, qs, w, k8, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0, gb, gr0); break;
    case 3: k_index_score_pf<FMT, 3, SC><<<grid, 256, 0, s>>>(q8, qs, w, k8, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0, gb, gr0); break;
    default: k_index_score_pf<FMT, 4, SC><<<grid, 256, 0, s>>>(q8, qs, w, k8, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0, gb, gr0); break;
  }
}

template <int FMT, typename SC>
static void dispatch_fmt(int DI, int QB, int HB, dim3 grid, hipStream_t s, const void* q, const void* qs,
                         const float* w, const void* kk, const void* ks, const int32_t* qp, int64_t Tq, int64_t N,
                         int H_I, int ratio, int64_t g0, int64_t gpb, int64_t ce, SC* sb, int64_t sr0, float* gb, int64_t gr0) {
  if constexpr (FMT == CSA_FP8_E4M3 || FMT == CSA_FP4_E2M1) {
    if (DI == 128 && QB == 4) {
      launch_score_pf<FMT, SC>(HB, grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0, gb, gr0);
      return;
    }
  }
  if (DI == 128) {
    if (QB == 4) dispatch_hb<FMT, 128, 4, SC>(HB, grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0, gb, gr0);
    else dispatch_hb<FMT, 128, 1, SC>(HB, grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0, gb, gr0);
  } else {
    if (QB == 4) dispatch_hb<FMT, 64, 4, SC>(HB, grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0, gb, gr0);
    else dispatch_hb<FMT, 64, 1, SC>(HB, grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0, gb, gr0);
  }
}

template <typename SC>
static hipError_t run_indexer(const void* q_idx, const void* q_scale, const float* w, const void* k_idx,
                              const void* k_scale, csa_dtype fmt, const int32_t* q_pos, int64_t B, int64_t Tq,
                              int64_t N, int H_I, int d_I, int ratio, int k, int32_t* idx_out, SC* score_out,
                              void* ws, hipStream_t s) {
  constexpr int SB = (int)sizeof(SC);
  const bool scores_only = idx_out == nullptr;   // the score stage alone, into score_out
  IndexPlan p = make_plan(B, Tq, N, SB, d_I, fmt, k);
  if (scores_only) p.lt = 0;
  const int HB = (H_I + 15) / 16;
  // group maxima and list composites follow the pass's score rows in the
  // workspace; the group maxima only when the selection reads them (rows
  // longer than kSmallN entries)
  uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
  float* gb = scores_only || N <= kSmallN ? nullptr : reinterpret_cast<float*>(wsb + score_area(p, N, SB));
  unsigned long long* lb =
      scores_only ? nullptr : reinterpret_cast<unsigned long long*>(wsb + score_area(p, N, SB) + group_area(p, N));
  for (int64_t g0 = 0; g0 < p.groups; g0 += p.groups_per_pass) {
    const int64_t g1 = (g0 + p.groups_per_pass) < p.groups ? (g0 + p.groups_per_pass) : p.groups;
    const int64_t rlo = (g0 / p.groups_per_batch) * Tq + (g0 % p.groups_per_batch) * p.QB;
    const int64_t glast = g1 - 1;
    int64_t rhi = (glast / p.groups_per_batch) * Tq + (glast % p.groups_per_batch) * p.QB + p.QB;
    const int64_t bend = (glast / p.groups_per_batch + 1) * Tq;
    if (rhi > bend) rhi = bend;
    SC* sb = score_out ? score_out : reinterpret_cast<SC*>(ws);
    const int64_t sr0 = score_out ? 0 : rlo;
    const int64_t gr0 = rlo;
    if (N > 0 && p.dec) {
      // one query per block row: rows rlo .. rlo + (g1 - g0)
      const dim3 grid((unsigned)p.dec_x, (unsigned)(g1 - g0));
      timer_before(CSA_KID_INDEX_SCORE, s);
      if (fmt == CSA_FP8_E4M3)
        launch_score_dec<CSA_FP8_E4M3, SC>(p.lt, HB, grid, s, q_idx, q_scale, w, k_idx, k_scale, q_pos, Tq, N, H_I, ratio, rlo, sb, sr0, gb, gr0, lb, rlo);
      else
        launch_score_dec<CSA_FP4_E2M1, SC>(p.lt, HB, grid, s, q_idx, q_scale, w, k_idx, k_scale, q_pos, Tq, N, H_I, ratio, rlo, sb, sr0, gb, gr0, lb, rlo);
      hipError_t e = hipGetLastError();
      timer_after(CSA_KID_INDEX_SCORE, s);
      if (e != hipSuccess) return e;
    } else if (N > 0) {
      const dim3 grid((unsigned)cdiv(N, p.chunk_entries), (unsigned)(g1 - g0));
      timer_before(CSA_KID_INDEX_SCORE, s);
      switch (fmt) {
        case CSA_FP8_E4M3: dispatch_fmt<CSA_FP8_E4M3, SC>(d_I, p.QB, HB, grid, s, q_idx, q_scale, w, k_idx, k_scale, q_pos, Tq, N, H_I, ratio, g0, p.groups_per_batch, p.chunk_entries, sb, sr0, gb, gr0); break;
        case CSA_FP4_E2M1: dispatch_fmt<CSA_FP4_E2M1, SC>(d_I, p.QB, HB, grid, s, q_idx, q_scale, w, k_idx, k_scale, q_pos, Tq, N, H_I, ratio, g0, p.groups_per_batch, p.chunk_entries, sb, sr0, gb, gr0); break;
        case CSA_BF16: dispatch_fmt<CSA_BF16, SC>(d_I, p.QB, HB, grid, s, q_idx, q_scale, w, k_idx, k_scale, q_pos, Tq, N, H_I, ratio, g0, p.groups_per_batch, p.chunk_entries, sb, sr0, gb, gr0); break;
        default: dispatch_fmt<CSA_F32, SC>(d_I, p.QB, HB, grid, s, q_idx, q_scale, w, k_idx, k_scale, q_pos, Tq, N, H_I, ratio, g0, p.groups_per_batch, p.chunk_entries, sb, sr0, gb, gr0); break;
      }
      hipError_t e = hipGetLastError();
      timer_after(CSA_KID_INDEX_SCORE, s);
      if (e != hipSuccess) return e;
    }
    if (scores_only) continue;
    const dim3 tgrid((unsigned)(rhi - rlo));
    timer_before(CSA_KID_TOPK, s);
    if (N <= kSmallN)   // every row is short: one 256-thread block per row
      k_topk_small<SC><<<tgrid, kSmallThreads, 0, s>>>(sb, sr0, rlo, q_pos, N, ratio, k, idx_out);
    else if (p.lt == 8)
      k_topk_lists<8, SC><<<tgrid, kTopkThreads, 0, s>>>(sb, sr0, lb, rlo, p.dec_x, rlo, q_pos, N, ratio, k, idx_out);
    else if (p.lt == 16)
      k_topk_lists<16, SC><<<tgrid, kTopkThreads, 0, s>>>(sb, sr0, lb, rlo, p.dec_x, rlo, q_pos, N, ratio, k, idx_out);
    else
      k_topk_select<SC><<<tgrid, kTopkThreads, 0, s>>>(sb, sr0, gb, gr0, rlo, q_pos, N, ratio, k, idx_out);
    hipError_t e = hipGetLastError();
    timer_after(CSA_KID_TOPK, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_indexer_scores(const void* q_idx, const void* q_scale, const float* w, const void* k_idx,
                                 const void* k_scale, csa_dtype fmt, const int32_t* q_pos, int64_t B, int64_t Tq,
                                 int64_t N, int H_I, int d_I, int ratio, float* score_out, hipStream_t s) {
  if (B * Tq == 0 || N == 0) return hipSuccess;
  return run_indexer<float>(q_idx, q_scale, w, k_idx, k_scale, fmt, q_pos, B, Tq, N, H_I, d_I, ratio, 1, nullptr,
                            score_out, nullptr, s);
}

hipError_t launch_indexer_topk(const void* q_idx, const void* q_scale, const float* w, const void* k_idx,
                               const void* k_scale, csa_dtype fmt, const int32_t* q_pos, int64_t B, int64_t Tq,
                               int64_t N, int H_I, int d_I, int ratio, int k, int32_t* idx_out, void* score_out,
                               bool bf16_scores, void* ws, hipStream_t s) {
  if (B * Tq == 0) return hipSuccess;
  if (bf16_scores)
    return run_indexer<uint16_t>(q_idx, q_scale, w, k_idx, k_scale, fmt, q_pos, B, Tq, N, H_I, d_I, ratio, k,
                                 idx_out, static_cast<uint16_t*>(score_out), ws, s);
  return run_indexer<float>(q_idx, q_scale, w, k_idx, k_scale, fmt, q_pos, B, Tq, N, H_I, d_I, ratio, k, idx_out,
                            static_cast<float*>(score_out), ws, s);
}

}  // namespace csa
