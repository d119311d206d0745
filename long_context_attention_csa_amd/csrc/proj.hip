// Projections around the attention core (cf-1.com write-up §3.4): the grouped
// output projection (heads split into groups, each group's concatenated head
// outputs reduced to a small rank, the group results concatenated and
// projected to the model width) and the indexer's query projection sharing the
// main attention's (one low-rank query latent feeding both the attention
// queries and the indexer queries). Both are chains of plain GEMMs, so they
// run on one hand-written bf16 MFMA GEMM:
//
//   C[g] (M x N) = A[g] (M x K) * W[g]^T        W[g]: N x K (a linear layer's
//                                               [out, in] weight), bf16 in,
//                                               float32 accumulation,
//                                               bf16 or float32 out,
// for g < G with element strides between the groups' A, W and C (groups of
// the output projection read column blocks of one A and write column blocks
// of one C).
//
// Kernel: a block computes a 128 x 128 tile of C with 4 waves (2 x 2, 64 x 64
// each, 4 x 4 tiles of v_mfma_f32_16x16x32_bf16), stepping K by 64 through a
// 2-slot LDS ring filled by global_load_lds_dwordx4 (each lane's 16 bytes
// straight to LDS). A tile row is 128 bytes, 8 chunks of 16. The MFMA's A
// operand is W (rows n) and its B operand is A (rows m): the accumulator
// then holds C^T, and a lane's 4 values are 4 consecutive
// columns of one row of C (one 8- or 16-byte store when C's rows are 16-byte
// aligned, else 4 element stores). Rows past M or N read the last valid row
// and are not stored; K is a multiple of 64. Problems with at least 256
// tiles of 256 x 256 (and M, N >= 256) use the large-tile kernel below (8 waves,
// 128 x 64 each); the chunk swizzle of both is c ^ ((r / 2) mod 8), which
// puts the 16 rows of a fragment read (two 128-byte rows per 256-byte bank
// line) on 16 different bank groups.
#include "attn_tile.hpp"

namespace csa {

constexpr int kGBM = 128, kGBN = 128, kGBK = 64;
constexpr int kGThreads = 256;
constexpr int kGLoads = kGBM * kGBK * 2 / 16 / kGThreads;   // 16-byte gathers per thread per operand tile (4)

template <bool OUT_BF16>
__global__ __launch_bounds__(kGThreads, 2) void k_gemm_bf16(const uint16_t* __restrict__ A, int64_t lda, int64_t sA,
                                                            const uint16_t* __restrict__ W, int64_t ldw, int64_t sW,
                                                            void* __restrict__ Cv, int64_t ldc, int64_t sC, int M,
                                                            int N, int K, int tiles_n, int vec_c) {
  __shared__ __align__(16) uint16_t sa[2][kGBM * kGBK];
  __shared__ __align__(16) uint16_t sw[2][kGBN * kGBK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, col = lane & 15;
  const int64_t grp = blockIdx.y;
  const int tile = blockIdx.x;
  const int m0 = (tile / tiles_n) * kGBM, n0 = (tile % tiles_n) * kGBN;
  A += grp * sA;
  W += grp * sW;
  const int wm = (wv & 1) * 64, wn = (wv >> 1) * 64;

  // Gather j of this lane: LDS bytes (4 j + wv) * 1024 + 16 lane, i.e. tile
  // row (4 j + wv) * 8 + lane / 8 at chunk position lane % 8, holding source
  // chunk (lane % 8) ^ (row % 8).
  const uint16_t* asrc[kGLoads];
  const uint16_t* wsrc[kGLoads];
#pragma unroll
  for (int j = 0; j < kGLoads; ++j) {
    const int row = (4 * j + wv) * 8 + (lane >> 3);
    const int ch = (lane & 7) ^ ((row >> 1) & 7);
    const int am = min(m0 + row, M - 1), wn_ = min(n0 + row, N - 1);
    asrc[j] = A + (int64_t)am * lda + 8 * ch;
    wsrc[j] = W + (int64_t)wn_ * ldw + 8 * ch;
  }
  auto issue = [&](int kt, int slot) {
    const int k0 = kt * kGBK;
#pragma unroll
    for (int j = 0; j < kGLoads; ++j) {
      gather_lds16(asrc[j] + k0, (uint32_t)(uintptr_t)(&sa[slot][0]) + (4 * j + wv) * 1024);
      gather_lds16(wsrc[j] + k0, (uint32_t)(uintptr_t)(&sw[slot][0]) + (4 * j + wv) * 1024);
    }
  };

  f32x4 acc[4][4];   // [n tile][m tile]: C^T blocks
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment read of tile row r (within the block tile), K chunk c: byte
  // r * 128 + 16 * (c ^ (r & 7))
  const int nk = K / kGBK;
  issue(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int slot = kt & 1;
    if (kt + 1 < nk) {
      issue(kt + 1, slot ^ 1);
      wait_vm<2 * kGLoads>();   // this step's gathers are done; the next step's stay in flight
    } else {
      wait_vm<0>();
    }
    __syncthreads();
    const uint32_t abase = (uint32_t)(uintptr_t)(&sa[slot][0]);
    const uint32_t wbase = (uint32_t)(uintptr_t)(&sw[slot][0]);
#pragma unroll
    for (int ks = 0; ks < kGBK / 32; ++ks) {
      const int c = 4 * ks + g;   // K chunk of this lane's 8 elements
      Frag<uint16_t> fa[4], fw[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int ra = wm + 16 * t + col, rw = wn + 16 * t + col;
        fa[t].v = lds_read_b128(abase + ra * 128 + 16 * (c ^ ((ra >> 1) & 7)));
        fw[t].v = lds_read_b128(wbase + rw * 128 + 16 * (c ^ ((rw >> 1) & 7)));
      }
#pragma unroll
      for (int tn = 0; tn < 4; ++tn)
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) acc[tn][tm] = mma8(fw[tn], fa[tm], acc[tn][tm]);
    }
    __syncthreads();   // the slot is refilled by the next issue
  }

  // acc[tn][tm][i] = C[m0 + wm + 16 tm + col][n0 + wn + 16 tn + 4 g + i]
#pragma unroll
  for (int tm = 0; tm < 4; ++tm) {
    const int m = m0 + wm + 16 * tm + col;
    if (m >= M) continue;
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
      const int n = n0 + wn + 16 * tn + 4 * g;
      if (n >= N) continue;
      const int64_t off = grp * sC + (int64_t)m * ldc + n;
      const f32x4 v = acc[tn][tm];
      if constexpr (OUT_BF16) {
        uint16_t* C = static_cast<uint16_t*>(Cv);
        if (vec_c && n + 4 <= N) {
          *reinterpret_cast<uint2*>(C + off) = make_uint2(cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3]));
        } else {
          for (int i = 0; i < 4 && n + i < N; ++i) C[off + i] = (uint16_t)(cvt_pk_bf16(v[i], 0.f) & 0xffffu);
        }
      } else {
        float* C = static_cast<float*>(Cv);
        if (vec_c && n + 4 <= N) {
          *reinterpret_cast<float4*>(C + off) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          for (int i = 0; i < 4 && n + i < N; ++i) C[off + i] = v[i];
        }
      }
    }
  }
}


// Large tiles: a block computes 256 x 256 of C with 8 waves (2 x 4, 128 x 64
// each: 8 x 4 tiles of v_mfma_f32_16x16x32_bf16, 128 accumulator registers),
// K step 64 through a 2-slot LDS ring (64 KB a slot). Twice the reuse of
// each staged element of the 128 x 128 kernel, so one block per compute unit
// keeps twice the bytes in flight per flop. Tiles are assigned so that the
// blocks one XCD runs (block b runs on XCD b mod 8) cover consecutive tiles,
// ordered in groups of 4 tile rows: neighbouring blocks of an XCD share A and
// W panels in its L2.
constexpr int kBM = 256, kBN = 256;
constexpr int kBThreads = 512;
constexpr int kBLoads = kBM * kGBK * 2 / 16 / kBThreads;   // 16-byte gathers per thread per operand tile (4)

__device__ __forceinline__ void big_tile_of(int b, int nblk, int tiles_m, int tiles_n, int& tm, int& tn) {
  // XCD-contiguous order: the blocks of XCD x (b mod 8 = x) take the x-th
  // of 8 consecutive ranges of tiles (the first nblk mod 8 ranges one longer)
  const int q = nblk >> 3, rem = nblk & 7, x = b & 7;
  const int t = x * q + min(x, rem) + (b >> 3);
  // groups of 4 tile rows, column-major inside a group
  const int gm = 4;
  const int group = t / (gm * tiles_n);
  const int first_m = group * gm;
  const int rows = min(gm, tiles_m - first_m);
  const int in = t - group * gm * tiles_n;
  tm = first_m + in % rows;
  tn = in / rows;
}

template <bool OUT_BF16>
__global__ __launch_bounds__(kBThreads, 1) void k_gemm_bf16_big(const uint16_t* __restrict__ A, int64_t lda, int64_t sA,
                                                             const uint16_t* __restrict__ W, int64_t ldw, int64_t sW,
                                                             void* __restrict__ Cv, int64_t ldc, int64_t sC, int M,
                                                             int N, int K, int tiles_m, int tiles_n, int vec_c) {
  __shared__ __align__(16) uint16_t sa[2 * kBM * kGBK];
  __shared__ __align__(16) uint16_t sw[2 * kBN * kGBK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, col = lane & 15;
  const int64_t grp = blockIdx.y;
  int tmi, tni;
  big_tile_of(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, tmi, tni);
  const int m0 = tmi * kBM, n0 = tni * kBN;
  A += grp * sA;
  W += grp * sW;
  const int wm = (wv & 1) * 128, wn = (wv >> 1) * 64;

  // Gather j of this lane: LDS bytes (8 j + wv) * 1024 + 16 lane, i.e. tile
  // row (8 j + wv) * 8 + lane / 8 at chunk position lane % 8, holding source
  // chunk (lane % 8) ^ ((row / 2) % 8).
  const uint16_t* asrc[kBLoads];
  const uint16_t* wsrc[kBLoads];
#pragma unroll
  for (int j = 0; j < kBLoads; ++j) {
    const int row = (8 * j + wv) * 8 + (lane >> 3);
    const int ch = (lane & 7) ^ ((row >> 1) & 7);
    const int am = min(m0 + row, M - 1), wn_ = min(n0 + row, N - 1);
    asrc[j] = A + (int64_t)am * lda + 8 * ch;
    wsrc[j] = W + (int64_t)wn_ * ldw + 8 * ch;
  }
  auto issue = [&](int kt, int slot) {
    const int k0 = kt * kGBK;
#pragma unroll
    for (int j = 0; j < kBLoads; ++j) {
      gather_lds16(asrc[j] + k0, (uint32_t)(uintptr_t)(sa + slot * kBM * kGBK) + (8 * j + wv) * 1024);
      gather_lds16(wsrc[j] + k0, (uint32_t)(uintptr_t)(sw + slot * kBN * kGBK) + (8 * j + wv) * 1024);
    }
  };

  f32x4 acc[4][8];   // [n tile][m tile]: C^T blocks
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / kGBK;
  issue(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int slot = kt & 1;
    if (kt + 1 < nk) {
      issue(kt + 1, slot ^ 1);
      wait_vm<2 * kBLoads>();   // this step's gathers are done; the next step's stay in flight
    } else {
      wait_vm<0>();
    }
    __syncthreads();
    const uint32_t abase = (uint32_t)(uintptr_t)(sa + slot * kBM * kGBK);
    const uint32_t wbase = (uint32_t)(uintptr_t)(sw + slot * kBN * kGBK);
#pragma unroll
    for (int ks = 0; ks < kGBK / 32; ++ks) {
      const int c = 4 * ks + g;   // K chunk of this lane's 8 elements
      Frag<uint16_t> fa[8], fw[4];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int ra = wm + 16 * t + col;
        fa[t].v = lds_read_b128(abase + ra * 128 + 16 * (c ^ ((ra >> 1) & 7)));
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int rw = wn + 16 * t + col;
        fw[t].v = lds_read_b128(wbase + rw * 128 + 16 * (c ^ ((rw >> 1) & 7)));
      }
#pragma unroll
      for (int tn = 0; tn < 4; ++tn)
#pragma unroll
        for (int tm = 0; tm < 8; ++tm) acc[tn][tm] = mma8(fw[tn], fa[tm], acc[tn][tm]);
    }
    __syncthreads();   // the slot is refilled by the next issue
  }

  // acc[tn][tm][i] = C[m0 + wm + 16 tm + col][n0 + wn + 16 tn + 4 g + i]
#pragma unroll
  for (int tm = 0; tm < 8; ++tm) {
    const int m = m0 + wm + 16 * tm + col;
    if (m >= M) continue;
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
      const int n = n0 + wn + 16 * tn + 4 * g;
      if (n >= N) continue;
      const int64_t off = grp * sC + (int64_t)m * ldc + n;
      const f32x4 v = acc[tn][tm];
      if constexpr (OUT_BF16) {
        uint16_t* C = static_cast<uint16_t*>(Cv);
        if (vec_c && n + 4 <= N) {
          *reinterpret_cast<uint2*>(C + off) = make_uint2(cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3]));
        } else {
          for (int i = 0; i < 4 && n + i < N; ++i) C[off + i] = (uint16_t)(cvt_pk_bf16(v[i], 0.f) & 0xffffu);
        }
      } else {
        float* C = static_cast<float*>(Cv);
        if (vec_c && n + 4 <= N) {
          *reinterpret_cast<float4*>(C + off) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          for (int i = 0; i < 4 && n + i < N; ++i) C[off + i] = v[i];
        }
      }
    }
  }
}

hipError_t launch_gemm_bf16(const void* A, int64_t lda, int64_t sA, const void* W, int64_t ldw, int64_t sW, void* C,
                            int64_t ldc, int64_t sC, int64_t M, int64_t N, int64_t K, int64_t G, bool out_bf16,
                            hipStream_t s) {
  if (M == 0 || N == 0 || G == 0) return hipSuccess;
  // 4-element vector stores when every row of C starts 16-byte aligned
  const int vec_c = (ldc % 4 == 0 && sC % 4 == 0 && ((uintptr_t)C & 15) == 0) ? 1 : 0;
  const int bm = (int)cdiv(M, kBM), bn = (int)cdiv(N, kBN);
  // large tiles when they fill the chip and are not mostly padding
  if ((int64_t)bm * bn * G >= 256 && M >= kBM && N >= kBN) {
    const dim3 grid((unsigned)(bm * bn), (unsigned)G);
    timer_before(CSA_KID_GEMM, s);
    if (out_bf16)
      k_gemm_bf16_big<true><<<grid, kBThreads, 0, s>>>(static_cast<const uint16_t*>(A), lda, sA,
                                                          static_cast<const uint16_t*>(W), ldw, sW, C, ldc, sC, (int)M,
                                                          (int)N, (int)K, bm, bn, vec_c);
    else
      k_gemm_bf16_big<false><<<grid, kBThreads, 0, s>>>(static_cast<const uint16_t*>(A), lda, sA,
                                                           static_cast<const uint16_t*>(W), ldw, sW, C, ldc, sC, (int)M,
                                                           (int)N, (int)K, bm, bn, vec_c);
    hipError_t e = hipGetLastError();
    timer_after(CSA_KID_GEMM, s);
    return e;
  }
  const int tiles_m = (int)cdiv(M, kGBM), tiles_n = (int)cdiv(N, kGBN);
  const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)G);
  timer_before(CSA_KID_GEMM, s);
  if (out_bf16)
    k_gemm_bf16<true><<<grid, kGThreads, 0, s>>>(static_cast<const uint16_t*>(A), lda, sA,
                                                 static_cast<const uint16_t*>(W), ldw, sW, C, ldc, sC, (int)M, (int)N,
                                                 (int)K, tiles_n, vec_c);
  else
    k_gemm_bf16<false><<<grid, kGThreads, 0, s>>>(static_cast<const uint16_t*>(A), lda, sA,
                                                  static_cast<const uint16_t*>(W), ldw, sW, C, ldc, sC, (int)M,
                                                  (int)N, (int)K, tiles_n, vec_c);
  hipError_t e = hipGetLastError();
  timer_after(CSA_KID_GEMM, s);
  return e;
}

}  // namespace csa
