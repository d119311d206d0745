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
// Select stage (k_topk_rows). One block per query row: a 13-bit histogram of
// the order-preserving score keys locates the bucket holding the k-th largest
// score; rows above it are taken, the bucket's members are resolved by a radix
// select on 64-bit (score key, inverted index) composites, which realises the
// total order "score descending, index ascending" exactly; the chosen indices
// are sorted ascending with a bitonic network. Deterministic by construction.
#include "common.hpp"

namespace csa {

constexpr int kTopkThreads = 512;
constexpr int kHistBits = 13;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kCandCap = kHistBins / 2;   // u64 candidates aliased onto the histogram
constexpr int kMaxK = 2048;

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
  i32x8 v;
  int scale;
  __device__ __forceinline__ void load(const uint8_t* row, const uint8_t* srow, int g) {
    if (DI == 128 || g < 2) {
      const i32x4 a = *reinterpret_cast<const i32x4*>(row + 16 * g);
      v = i32x8{a[0], a[1], a[2], a[3], 0, 0, 0, 0};
      scale = srow[g];
    } else {
      v = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
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
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a.v, b.v, acc, 4, 4, 0, a.scale, 0, b.scale);
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

// ------------------------------------------------------------------ score kernel
// grid.x: entry chunk (chunk_entries entries each), grid.y: query group
// (QB consecutive queries of one sequence), 256 threads (4 waves).
// Group gy covers rows row_lo(gy) .. ; row r writes scores at sbase + (r - srow0) * N.
template <int FMT, int DI, int HB, int QB>
__global__ __launch_bounds__(256) void k_index_score(
    const void* __restrict__ q_idx, const void* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ k_idx, const void* __restrict__ k_scale, const int32_t* __restrict__ q_pos,
    int64_t Tq, int64_t N, int H_I, int ratio, int64_t group0, int64_t groups_per_batch,
    int64_t chunk_entries, float* __restrict__ sbase, int64_t srow0) {
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
        if constexpr (FMT == CSA_FP8_E4M3 || FMT == CSA_FP4_E2M1) qa[qi][hb].v = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
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
  for (int64_t e0 = e_begin + 16 * wv; e0 < e_end; e0 += 64) {
    const int64_t e = e0 + col;
    const int64_t esafe = e < N ? e : N - 1;
    Operand<FMT, DI> kb;
    if constexpr (FMT == CSA_FP4_E2M1)
      kb.load(kbase + esafe * RU, reinterpret_cast<const uint8_t*>(k_scale) + (b * N + esafe) * (DI / 32), g);
    else
      kb.load(kbase + esafe * RU, g);
    float ks = 1.f;
    if constexpr (FMT == CSA_FP8_E4M3) ks = reinterpret_cast<const float*>(k_scale)[b * N + esafe];
#pragma unroll
    for (int qi = 0; qi < QB; ++qi) {
      if (qi >= nq) break;
      float part = 0.f;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const f32x4 acc = mma_tile<FMT, DI>(qa[qi][hb], kb);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) part = fmaf(wq[qi][hb][rr], fmaxf(acc[rr], 0.f), part);
      }
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      if constexpr (FMT == CSA_FP8_E4M3) part *= ks;
      if (g == 0 && e < nvis[qi]) {
        const int64_t r = b * Tq + t0 + qi;
        sbase[(r - srow0) * N + e] = part;
      }
    }
  }
}

// ------------------------------------------------------------------ block helpers

// Inclusive scan across the block of one value per thread (kTopkThreads threads).
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  if (lane == 63) wsum[wv] = v;
  __syncthreads();
  uint32_t add = 0;
  for (int i = 0; i < wv; ++i) add += wsum[i];
  __syncthreads();
  return v + add;
}

// Top-k of one row of scores (n entries, keff = min(k, n) > 0 entries wanted,
// n > k). Writes the ascending selection into sel[0..keff).
struct TopkSmem {
  union {
    uint32_t hist[kHistBins];
    unsigned long long cand[kCandCap];
  };
  int sel[kMaxK];
  uint32_t h256[256];
  uint32_t wsum[16];
  int nsel, ncand;
  uint32_t d1, need;
  unsigned long long prefix, mask, thresh;
  int done;
};

__device__ __forceinline__ unsigned long long composite(uint32_t key, int64_t i) {
  return ((unsigned long long)key << 32) | (unsigned long long)(0xffffffffu - (uint32_t)i);
}

// Radix select: the need-th largest composite among alive elements
// (those whose masked bits equal the prefix). get(i) -> (valid, key64).
template <typename Get>
__device__ void radix_threshold(TopkSmem& sm, int64_t count, Get get) {
  const int tid = threadIdx.x;
  int shift = 64;
  // bits already fixed: the mask's leading ones
  for (;;) {
    // next digit: up to 8 bits directly below the fixed bits
    const int fixed = __popcll(sm.mask);
    const int width = (64 - fixed) < 8 ? (64 - fixed) : 8;
    shift = 64 - fixed - width;
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
    if (tid == 0) {
      uint32_t need = sm.need, above = 0;
      int dd = (1 << width) - 1;
      for (; dd > 0; --dd) {
        if (above + sm.h256[dd] >= need) break;
        above += sm.h256[dd];
      }
      need -= above;
      sm.prefix = prefix | ((unsigned long long)dd << shift);
      sm.mask = mask | dmask;
      sm.need = need;
      sm.done = (sm.h256[dd] == need) || (sm.mask == ~0ull);
      sm.thresh = sm.prefix;   // remaining low bits zero: key >= thresh <=> chosen
    }
    __syncthreads();
    if (sm.done) break;
  }
}

__device__ void bitonic_sort_sel(TopkSmem& sm, int keff) {
  int P = 1;
  while (P < keff) P <<= 1;
  for (int i = keff + threadIdx.x; i < P; i += kTopkThreads) sm.sel[i] = 0x7fffffff;
  __syncthreads();
  for (int k2 = 2; k2 <= P; k2 <<= 1) {
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < P; i += kTopkThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const int a = sm.sel[i], c = sm.sel[ixj];
          const bool up = (i & k2) == 0;
          if ((a > c) == up) { sm.sel[i] = c; sm.sel[ixj] = a; }
        }
      }
      __syncthreads();
    }
  }
}

// One block per row of the current chunk. Scores of row r live at
// sbase + (r - srow0) * N.
__global__ __launch_bounds__(kTopkThreads) void k_topk_rows(const float* __restrict__ sbase, int64_t srow0,
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
  const int keff = k;
  const float* srow = sbase + (r - srow0) * N;

  // Pass 1: 13-bit histogram of the order keys.
  for (int i = tid; i < kHistBins; i += kTopkThreads) sm.hist[i] = 0;
  if (tid == 0) { sm.nsel = 0; sm.ncand = 0; }
  __syncthreads();
  for (int64_t i = tid; i < n; i += kTopkThreads) atomicAdd(&sm.hist[order_key(srow[i]) >> (32 - kHistBits)], 1u);
  __syncthreads();
  // Locate the bucket of the keff-th largest: thread t owns 16 bins from the top.
  constexpr int BPT = kHistBins / kTopkThreads;
  const int top = kHistBins - BPT * tid;   // owns bins [top - BPT, top)
  uint32_t mine = 0;
#pragma unroll
  for (int i = 1; i <= BPT; ++i) mine += sm.hist[top - i];
  const uint32_t incl = block_inclusive_scan(mine, sm.wsum);
  const uint32_t excl = incl - mine;
  if (excl < (uint32_t)keff && incl >= (uint32_t)keff) {
    uint32_t above = excl;
    int bin = top - 1;
    for (; bin > top - BPT; --bin) {
      if (above + sm.hist[bin] >= (uint32_t)keff) break;
      above += sm.hist[bin];
    }
    sm.d1 = (uint32_t)bin;
    sm.need = (uint32_t)keff - above;
  }
  __syncthreads();
  const uint32_t d1 = sm.d1;

  // Pass 2: take rows above the bucket, collect the bucket's members.
  for (int64_t i = tid; i < n; i += kTopkThreads) {
    const uint32_t key = order_key(srow[i]);
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
  if ((uint32_t)ncand == sm.need) {
    for (int c = tid; c < ncand; c += kTopkThreads)
      sm.sel[atomicAdd(&sm.nsel, 1)] = (int)(0xffffffffu - (uint32_t)(sm.cand[c] & 0xffffffffu));
  } else if (ncand <= kCandCap) {
    radix_threshold(sm, ncand, [&](int64_t i, bool& ok) { ok = true; return sm.cand[i]; });
    const unsigned long long th = sm.thresh;
    for (int c = tid; c < ncand; c += kTopkThreads)
      if (sm.cand[c] >= th) sm.sel[atomicAdd(&sm.nsel, 1)] = (int)(0xffffffffu - (uint32_t)(sm.cand[c] & 0xffffffffu));
  } else {
    // Bucket larger than the LDS list (heavy ties): select straight from the row.
    radix_threshold(sm, n, [&](int64_t i, bool& ok) {
      ok = true;
      return composite(order_key(srow[i]), i);
    });
    const unsigned long long th = sm.thresh;
    for (int64_t i = tid; i < n; i += kTopkThreads) {
      const uint32_t key = order_key(srow[i]);
      if ((key >> (32 - kHistBits)) == d1 && composite(key, i) >= th) sm.sel[atomicAdd(&sm.nsel, 1)] = (int)i;
    }
  }
  __syncthreads();
  bitonic_sort_sel(sm, keff);
  for (int i = tid; i < k; i += kTopkThreads) out[i] = i < keff ? sm.sel[i] : -1;
}

// ------------------------------------------------------------------ host side

struct IndexPlan {
  int QB;
  int64_t groups_per_batch, groups, chunk_entries, groups_per_pass, max_rows_per_pass;
};

static IndexPlan make_plan(int64_t B, int64_t Tq, int64_t N) {
  IndexPlan p;
  p.QB = Tq >= 4 ? 4 : 1;
  p.groups_per_batch = cdiv(Tq, p.QB);
  p.groups = B * p.groups_per_batch;
  // Enough blocks to cover the chip several times: split entries when groups are few.
  const int64_t want_blocks = 2048;
  int64_t chunks = cdiv(want_blocks, p.groups);
  const int64_t max_chunks = cdiv(N, 256);
  if (chunks > max_chunks) chunks = max_chunks;
  if (chunks < 1) chunks = 1;
  p.chunk_entries = cdiv(cdiv(N, chunks), 64) * 64;
  if (p.chunk_entries < 64) p.chunk_entries = 64;
  // Score buffer budget per pass: 1 GiB.
  const int64_t budget = (int64_t)1 << 30;
  const int64_t row_bytes = (N > 0 ? N : 1) * 4;
  int64_t gpp = budget / (row_bytes * p.QB);
  if (gpp < 1) gpp = 1;
  if (gpp > 65535) gpp = 65535;
  if (gpp > p.groups) gpp = p.groups;
  p.groups_per_pass = gpp;
  p.max_rows_per_pass = gpp * p.QB;
  return p;
}

size_t indexer_ws_bytes(int64_t B, int64_t Tq, int64_t N) {
  const IndexPlan p = make_plan(B, Tq, N);
  return (size_t)p.max_rows_per_pass * (size_t)N * 4 + 256;
}

template <int FMT, int DI, int HB, int QB>
static void launch_score(dim3 grid, hipStream_t s, const void* q, const void* qs, const float* w, const void* kk,
                         const void* ks, const int32_t* qp, int64_t Tq, int64_t N, int H_I, int ratio, int64_t g0,
                         int64_t gpb, int64_t ce, float* sb, int64_t sr0) {
  k_index_score<FMT, DI, HB, QB><<<grid, 256, 0, s>>>(q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0);
}

template <int FMT, int DI, int QB>
static void dispatch_hb(int HB, dim3 grid, hipStream_t s, const void* q, const void* qs, const float* w,
                        const void* kk, const void* ks, const int32_t* qp, int64_t Tq, int64_t N, int H_I,
                        int ratio, int64_t g0, int64_t gpb, int64_t ce, float* sb, int64_t sr0) {
  switch (HB) {
    case 1: launch_score<FMT, DI, 1, QB>(grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0); break;
    case 2: launch_score<FMT, DI, 2, QB>(grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0); break;
    case 3: launch_score<FMT, DI, 3, QB>(grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0); break;
    default: launch_score<FMT, DI, 4, QB>(grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0); break;
  }
}

template <int FMT>
static void dispatch_fmt(int DI, int QB, int HB, dim3 grid, hipStream_t s, const void* q, const void* qs,
                         const float* w, const void* kk, const void* ks, const int32_t* qp, int64_t Tq, int64_t N,
                         int H_I, int ratio, int64_t g0, int64_t gpb, int64_t ce, float* sb, int64_t sr0) {
  if (DI == 128) {
    if (QB == 4) dispatch_hb<FMT, 128, 4>(HB, grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0);
    else dispatch_hb<FMT, 128, 1>(HB, grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0);
  } else {
    if (QB == 4) dispatch_hb<FMT, 64, 4>(HB, grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0);
    else dispatch_hb<FMT, 64, 1>(HB, grid, s, q, qs, w, kk, ks, qp, Tq, N, H_I, ratio, g0, gpb, ce, sb, sr0);
  }
}

hipError_t launch_indexer_topk(const void* q_idx, const void* q_scale, const float* w, const void* k_idx,
                               const void* k_scale, csa_dtype fmt, const int32_t* q_pos, int64_t B, int64_t Tq,
                               int64_t N, int H_I, int d_I, int ratio, int k, int32_t* idx_out, float* score_out,
                               void* ws, hipStream_t s) {
  if (B * Tq == 0) return hipSuccess;
  const IndexPlan p = make_plan(B, Tq, N);
  const int HB = (H_I + 15) / 16;
  for (int64_t g0 = 0; g0 < p.groups; g0 += p.groups_per_pass) {
    const int64_t g1 = (g0 + p.groups_per_pass) < p.groups ? (g0 + p.groups_per_pass) : p.groups;
    const int64_t rlo = (g0 / p.groups_per_batch) * Tq + (g0 % p.groups_per_batch) * p.QB;
    const int64_t glast = g1 - 1;
    int64_t rhi = (glast / p.groups_per_batch) * Tq + (glast % p.groups_per_batch) * p.QB + p.QB;
    const int64_t bend = (glast / p.groups_per_batch + 1) * Tq;
    if (rhi > bend) rhi = bend;
    float* sb = score_out ? score_out : reinterpret_cast<float*>(ws);
    const int64_t sr0 = score_out ? 0 : rlo;
    if (N > 0) {
      const dim3 grid((unsigned)cdiv(N, p.chunk_entries), (unsigned)(g1 - g0));
      timer_before(CSA_KID_INDEX_SCORE, s);
      switch (fmt) {
        case CSA_FP8_E4M3: dispatch_fmt<CSA_FP8_E4M3>(d_I, p.QB, HB, grid, s, q_idx, q_scale, w, k_idx, k_scale, q_pos, Tq, N, H_I, ratio, g0, p.groups_per_batch, p.chunk_entries, sb, sr0); break;
        case CSA_FP4_E2M1: dispatch_fmt<CSA_FP4_E2M1>(d_I, p.QB, HB, grid, s, q_idx, q_scale, w, k_idx, k_scale, q_pos, Tq, N, H_I, ratio, g0, p.groups_per_batch, p.chunk_entries, sb, sr0); break;
        case CSA_BF16: dispatch_fmt<CSA_BF16>(d_I, p.QB, HB, grid, s, q_idx, q_scale, w, k_idx, k_scale, q_pos, Tq, N, H_I, ratio, g0, p.groups_per_batch, p.chunk_entries, sb, sr0); break;
        default: dispatch_fmt<CSA_F32>(d_I, p.QB, HB, grid, s, q_idx, q_scale, w, k_idx, k_scale, q_pos, Tq, N, H_I, ratio, g0, p.groups_per_batch, p.chunk_entries, sb, sr0); break;
      }
      hipError_t e = hipGetLastError();
      timer_after(CSA_KID_INDEX_SCORE, s);
      if (e != hipSuccess) return e;
    }
    timer_before(CSA_KID_TOPK, s);
    k_topk_rows<<<dim3((unsigned)(rhi - rlo)), kTopkThreads, 0, s>>>(sb, sr0, rlo, q_pos, N, ratio, k, idx_out);
    hipError_t e = hipGetLastError();
    timer_after(CSA_KID_TOPK, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace csa
