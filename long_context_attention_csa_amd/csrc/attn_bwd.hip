// Backward of the core attention of CSA (selected compressed entries) and HCA
// (all visible entries), each joined with the window and the sink; bf16
// operands, float32 accumulation.
//
// cf-1.com write-up §4.3: training runs a deterministic attention backward
// (the write-up gives each streaming multiprocessor its own accumulation
// buffer). The pages print no formulas; these are the gradients of the
// forward's definition (§3.1-§3.3). For query row r, head h and key i of the
// row's key set (keys are also values; the sink is one more softmax term
// with no value):
//   P_hi = exp(l_hi - lse_h),  l_hi = scale q_h . K_i,
//   D_h = dO_h . O_h,  dP_hi = dO_h . K_i,  dl_hi = P_hi (dP_hi - D_h),
//   dq_h   = scale sum_i dl_hi K_i,
//   dK_i  += sum_h (scale dl_hi q_h + P_hi dO_h),
//   dsink_h += -exp(sink_h - lse_h) D_h.
//
// Determinism without float atomics: each (query, key slot) writes its key
// row gradient G (128 float32) exactly once, at a position given by an
// inverted selection in which the slots of each key follow one fixed order
// (query chunk, then query within the chunk); a reduction then adds each
// key's contributions in that order. Instead of per-compute-unit buffers of
// all N rows (read-modify-written by every query), the buffer holds only the
// contributions, written once and read once, and its size does not grow
// with N. Query rows are processed in passes whose contributions fit a fixed
// budget; later passes add to the earlier sums in pass order.
//
// Kernels of one pass (one stream, in order):
//   k_fill_u32         clear the per-chunk key counters
//   k_bwd_count        counters[chunk][key] += 1 per (query, slot)
//   k_bwd_chunk_scan   per key: exclusive prefix over chunks, and the total
//   k_bwd_scan_*       exclusive prefix of the totals over keys: list offsets
//   k_bwd_place        per chunk, query by query: the position of each slot
//   k_attn_bwd16       per query: dq, the slot gradients G, the sink terms
//                      (D = dO . O per row and head comes from k_bwd_delta, run
//                      once before the passes)
//   k_bwd_reduce       per key: sum of its contributions in list order
// Dense layers take contributions for their window rows only; the entries'
// gradients come from k_attn_bwd_dense_kv (per block of entries and segment
// of query rows, summed in registers) and k_bwd_seg_reduce.
// and once at the end k_bwd_sink_part / k_bwd_sink_final (sink gradient over
// all rows in a fixed order).
#include "attn_tile.hpp"

namespace csa {

constexpr int kBwdThreads = 256;
constexpr int kBwdQc = 64;                       // query rows per placement chunk
constexpr int64_t kBwdGBudget = (int64_t)4 << 30;   // bytes of G per pass
constexpr int kScanPer = 16;                     // totals per thread in the key scan
constexpr int kScanBlock = kBwdThreads * kScanPer;
constexpr int kSinkBlocks = 256;                 // first-level blocks of the sink gradient sum

// Key set of a query row: n_sel selected (or visible) slots, then n_win
// window rows starting at absolute position lo.
struct BwdRow {
  int64_t b, w0, n_sel, lo, n_win;
};

template <bool SPARSE>
__device__ __forceinline__ BwdRow bwd_row(int64_t r, int64_t Tq, int64_t N, int64_t T_win, int k, int window,
                                          int ratio, const int32_t* __restrict__ win_start,
                                          const int32_t* __restrict__ q_pos) {
  BwdRow w;
  w.b = r / Tq;
  const int32_t p = q_pos[r];
  w.w0 = win_start[w.b];
  w.n_sel = SPARSE ? (int64_t)k : visible(p, ratio, N);
  int64_t lo = (int64_t)p - window + 1;
  if (lo < 0) lo = 0;
  if (lo < w.w0) lo = w.w0;
  int64_t hi = p;
  if (hi > w.w0 + T_win - 1) hi = w.w0 + T_win - 1;
  w.lo = lo;
  w.n_win = (window > 0 && hi >= lo) ? hi - lo + 1 : 0;
  return w;
}

// Key id of slot j (< n_sel + n_win): entry e of batch b is b (N + T_win) + e,
// window row t is b (N + T_win) + N + t; -1 for a slot without a key.
// Dense layers count window slots only, with ids b T_win + t (their entries'
// gradients come from k_attn_bwd_dense_kv).
template <bool SPARSE>
__device__ __forceinline__ int64_t bwd_slot_id(const BwdRow& w, const int32_t* __restrict__ idx, int64_t r, int k,
                                               int64_t N, int64_t T_win, int64_t j) {
  if (!SPARSE) return j < w.n_sel ? -1 : w.b * T_win + (w.lo + (j - w.n_sel) - w.w0);
  const int64_t base = w.b * (N + T_win);
  if (j < w.n_sel) {
    const int64_t e = SPARSE ? (int64_t)idx[r * k + j] : j;
    return (e >= 0 && e < N) ? base + e : -1;
  }
  return base + N + (w.lo + (j - w.n_sel) - w.w0);
}

__global__ __launch_bounds__(kBwdThreads) void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * kBwdThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBwdThreads)
    p[i] = v;
}

template <bool SPARSE>
__global__ __launch_bounds__(kBwdThreads) void k_bwd_count(const int32_t* __restrict__ idx,
                                                           const int32_t* __restrict__ win_start,
                                                           const int32_t* __restrict__ q_pos, int64_t r0, int64_t Tq,
                                                           int64_t N, int64_t T_win, int k, int window, int ratio,
                                                           int64_t nids, uint32_t* __restrict__ cnt) {
  const int64_t r = r0 + blockIdx.x;
  const BwdRow w = bwd_row<SPARSE>(r, Tq, N, T_win, k, window, ratio, win_start, q_pos);
  uint32_t* c = cnt + (int64_t)(blockIdx.x / kBwdQc) * nids;
  const int64_t nk = w.n_sel + w.n_win;
  for (int64_t j = (SPARSE ? 0 : w.n_sel) + threadIdx.x; j < nk; j += kBwdThreads) {
    const int64_t id = bwd_slot_id<SPARSE>(w, idx, r, k, N, T_win, j);
    if (id >= 0) atomicAdd(c + id, 1u);
  }
}

// Per key: counters[c] <- sum of counters[c' < c]; total <- sum over chunks.
__global__ __launch_bounds__(kBwdThreads) void k_bwd_chunk_scan(uint32_t* __restrict__ cnt, int64_t nids,
                                                                int nchunks, uint32_t* __restrict__ total) {
  const int64_t id = (int64_t)blockIdx.x * kBwdThreads + threadIdx.x;
  if (id >= nids) return;
  uint32_t run = 0;
  for (int c = 0; c < nchunks; ++c) {
    const uint32_t v = cnt[c * nids + id];
    cnt[c * nids + id] = run;
    run += v;
  }
  total[id] = run;
}

// Exclusive scan of v over the block (256 threads); returns the block total in *tot.
__device__ __forceinline__ uint32_t bwd_block_scan(uint32_t v, uint32_t* wsum, uint32_t* tot) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kBwdThreads / 64; ++i) {
    before += i < wv ? wsum[i] : 0u;
    all += wsum[i];
  }
  __syncthreads();
  *tot = all;
  return before + x - v;
}

__global__ __launch_bounds__(kBwdThreads) void k_bwd_scan_sums(const uint32_t* __restrict__ total, int64_t n,
                                                               uint32_t* __restrict__ bsum) {
  __shared__ uint32_t wsum[kBwdThreads / 64];
  const int64_t i0 = (int64_t)blockIdx.x * kScanBlock + (int64_t)threadIdx.x * kScanPer;
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) s += (i0 + j < n) ? total[i0 + j] : 0u;
  uint32_t tot;
  (void)bwd_block_scan(s, wsum, &tot);
  if (threadIdx.x == 0) bsum[blockIdx.x] = tot;
}

// One block: exclusive scan of the nb block sums in place (in rounds of 256).
__global__ __launch_bounds__(kBwdThreads) void k_bwd_scan_top(uint32_t* __restrict__ bsum, int64_t nb) {
  __shared__ uint32_t wsum[kBwdThreads / 64];
  uint32_t carry = 0;
  for (int64_t base = 0; base < nb; base += kBwdThreads) {
    const int64_t i = base + threadIdx.x;
    const uint32_t v = i < nb ? bsum[i] : 0u;
    uint32_t tot;
    const uint32_t ex = bwd_block_scan(v, wsum, &tot);
    if (i < nb) bsum[i] = carry + ex;
    carry += tot;
  }
}

// off[i] = exclusive prefix of total at i; off[n] = the sum of all.
__global__ __launch_bounds__(kBwdThreads) void k_bwd_scan_apply(const uint32_t* __restrict__ total, int64_t n,
                                                                const uint32_t* __restrict__ bsum,
                                                                uint32_t* __restrict__ off) {
  __shared__ uint32_t wsum[kBwdThreads / 64];
  const int64_t i0 = (int64_t)blockIdx.x * kScanBlock + (int64_t)threadIdx.x * kScanPer;
  uint32_t v[kScanPer];
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) {
    v[j] = (i0 + j < n) ? total[i0 + j] : 0u;
    s += v[j];
  }
  uint32_t tot;
  uint32_t run = bsum[blockIdx.x] + bwd_block_scan(s, wsum, &tot);
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) {
    if (i0 + j < n) off[i0 + j] = run;
    run += v[j];
    if (i0 + j == n - 1) off[n] = run;
  }
}

// One block per chunk of kBwdQc query rows, taken one query at a time: each
// slot takes the next position of its key's range in the chunk. Slots of one
// query have distinct keys (a repeated selected entry gets two positions,
// whose contributions are equal), and the barrier orders the queries.
template <bool SPARSE>
__global__ __launch_bounds__(kBwdThreads) void k_bwd_place(const int32_t* __restrict__ idx,
                                                           const int32_t* __restrict__ win_start,
                                                           const int32_t* __restrict__ q_pos, int64_t r0, int64_t r1,
                                                           int64_t Tq, int64_t N, int64_t T_win, int k, int window,
                                                           int ratio, int64_t nids, uint32_t* __restrict__ cnt,
                                                           const uint32_t* __restrict__ off,
                                                           int32_t* __restrict__ posbuf, int64_t smax) {
  const int64_t rc0 = r0 + (int64_t)blockIdx.x * kBwdQc;
  uint32_t* c = cnt + (int64_t)blockIdx.x * nids;
  for (int qi = 0; qi < kBwdQc; ++qi) {
    const int64_t r = rc0 + qi;
    if (r >= r1) break;
    const BwdRow w = bwd_row<SPARSE>(r, Tq, N, T_win, k, window, ratio, win_start, q_pos);
    const int64_t nk = w.n_sel + w.n_win;
    const int64_t j0 = SPARSE ? 0 : w.n_sel;   // dense rows list window slots only
    int32_t* prow = posbuf + (r - r0) * smax - j0;
    for (int64_t j = j0 + threadIdx.x; j < nk; j += kBwdThreads) {
      const int64_t id = bwd_slot_id<SPARSE>(w, idx, r, k, N, T_win, j);
      prow[j] = id >= 0 ? (int32_t)(off[id] + atomicAdd(c + id, 1u)) : -1;
    }
    __syncthreads();
  }
}


// Swizzle of the 8-byte units of a P / dl row (64 keys, 128 bytes): unit u of
// row x sits at u ^ pdl_swz(x & 15), the row's two 2-bit halves swapped. The
// writes (16 consecutive rows, one unit) and the transposed reads (4
// consecutive rows x 4 adjacent units) then each touch 16 distinct units.
__device__ __forceinline__ int pdl_swz(int x) { return ((x & 3) << 2) | ((x >> 2) & 3); }

// 8-byte LDS store at a byte address.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2;
__device__ __forceinline__ void lds_write_b64(uint32_t a, uint32_t lo, uint32_t hi) {
  *(lds_u32x2*)(size_t)a = u32x2_t{lo, hi};
}

// P and scale * dl of a lane (head h0 + 16 hb + col, keys 16 kb + 4 g .. + 3)
// into the [head][key] tiles at plb / dlb.
template <int HPW>
__device__ __forceinline__ void write_pdl(uint32_t plb, uint32_t dlb, int h0, int g, int col,
                                          const float (&s)[HPW][4][4], const float (&dp)[HPW][4][4]) {
#pragma unroll
  for (int hb = 0; hb < HPW; ++hb) {
    const int hh = h0 + 16 * hb + col;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint32_t o = (uint32_t)hh * 128u + 8u * (uint32_t)((4 * kb + g) ^ pdl_swz(hh & 15));
      lds_write_b64(plb + o, cvt_pk_bf16(s[hb][kb][0], s[hb][kb][1]), cvt_pk_bf16(s[hb][kb][2], s[hb][kb][3]));
      lds_write_b64(dlb + o, cvt_pk_bf16(dp[hb][kb][0], dp[hb][kb][1]), cvt_pk_bf16(dp[hb][kb][2], dp[hb][kb][3]));
    }
  }
}

// acc += G^T = Q^T (scale dl) + dO^T P for the wave's d blocks 2 wv, 2 wv + 1
// and the 4 key blocks of a 64-key tile; K runs over the H heads, 32 per step.
// ga / gb: the lane's tile-invariant transposed-read offsets.
template <int H>
__device__ __forceinline__ void gt_accum(f32x4 (&acc)[2][4], uint32_t qtb, uint32_t otb, uint32_t plb, uint32_t dlb,
                                         const uint32_t (&ga)[2], const uint32_t (&gb)[4]) {
#pragma unroll
  for (int ks = 0; ks < H / 32; ++ks) {
    Frag<uint16_t> aq[2], ao[2];
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2) {
      const uint32_t a = ga[d2] + 8192u * (uint32_t)ks;
      const i32x2 q0 = __builtin_bit_cast(i32x2, lds_read_tr16(qtb + a));
      const i32x2 q1 = __builtin_bit_cast(i32x2, lds_read_tr16(qtb + a + 4096));
      const i32x2 o0 = __builtin_bit_cast(i32x2, lds_read_tr16(otb + a));
      const i32x2 o1 = __builtin_bit_cast(i32x2, lds_read_tr16(otb + a + 4096));
      aq[d2].v = i32x4{q0[0], q0[1], q1[0], q1[1]};
      ao[d2].v = i32x4{o0[0], o0[1], o1[0], o1[1]};
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      // rows 32 ks + trow (+ 16) share the swizzle of row trow
      const uint32_t olo = gb[nb] + 4096u * (uint32_t)ks, ohi = olo + 2048u;
      const i32x2 l0 = __builtin_bit_cast(i32x2, lds_read_tr16(dlb + olo));
      const i32x2 l1 = __builtin_bit_cast(i32x2, lds_read_tr16(dlb + ohi));
      const i32x2 p0 = __builtin_bit_cast(i32x2, lds_read_tr16(plb + olo));
      const i32x2 p1 = __builtin_bit_cast(i32x2, lds_read_tr16(plb + ohi));
      Frag<uint16_t> bl, bp;
      bl.v = i32x4{l0[0], l0[1], l1[0], l1[1]};
      bp.v = i32x4{p0[0], p0[1], p1[0], p1[1]};
#pragma unroll
      for (int d2 = 0; d2 < 2; ++d2) {
        acc[d2][nb] = mma8(aq[d2], bl, acc[d2][nb]);
        acc[d2][nb] = mma8(ao[d2], bp, acc[d2][nb]);
      }
    }
  }
}

// The lane's tile-invariant offsets for gt_accum: transposed reads of the
// Q / dO rows for d blocks 2 wv, 2 wv + 1, and of P / dl for key block nb
// (row trow = 4 g + col / 4 of each 16-row block, unit 4 nb + col % 4).
__device__ __forceinline__ void gt_offsets(const TileLanes& tl, int wv, int g, int col, uint32_t (&ga)[2],
                                           uint32_t (&gb)[4]) {
#pragma unroll
  for (int d2 = 0; d2 < 2; ++d2) {
    ga[d2] = (((uint32_t)(32 * (2 * wv + d2))) ^ tl.vx) + tl.vofs;
    opaque(ga[d2]);
  }
  const int trow = 4 * g + (col >> 2);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    gb[nb] = (uint32_t)trow * 128u + 8u * (uint32_t)((4 * nb + (col & 3)) ^ pdl_swz(trow));
    opaque(gb[nb]);
  }
}

// D[r, h] = dO[r, h] . O[r, h] for every (row, head): 16 lanes per pair,
// 8 elements each, summed over the 16 lanes by xor-shuffles (fixed order).
__global__ __launch_bounds__(kBwdThreads) void k_bwd_delta(const uint16_t* __restrict__ out,
                                                           const uint16_t* __restrict__ dout, int64_t pairs,
                                                           float* __restrict__ D) {
  const int64_t pr = (int64_t)blockIdx.x * (kBwdThreads / 16) + (threadIdx.x >> 4);
  const int l = threadIdx.x & 15;
  float acc = 0.f;
  if (pr < pairs) {
    const i32x4 a = *reinterpret_cast<const i32x4*>(dout + pr * kD + 8 * l);
    const i32x4 o = *reinterpret_cast<const i32x4*>(out + pr * kD + 8 * l);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(__uint_as_float((uint32_t)a[e] << 16), __uint_as_float((uint32_t)o[e] << 16), acc);
      acc = fmaf(__uint_as_float((uint32_t)a[e] & 0xffff0000u), __uint_as_float((uint32_t)o[e] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) acc += __shfl_xor(acc, m);
  if (pr < pairs && l == 0) D[pr] = acc;
}

// One block per query row, 4 waves; H = 64 HPW heads, wave w owns heads
// [16 HPW w, 16 HPW (w + 1)) for the products over d and the d blocks
// {2w, 2w + 1} of the key-row gradients. Per 64-key tile:
//   S^T = K Q^T, dP^T = K dO^T        A = key rows (LDS), B = Q, dO (registers)
//   P, dl                             per head = per lane column
//   dQ^T += K^T dl^T                  A = transposed key-tile reads, B = dl
//   P, dl -> LDS as [head][key]
//   G^T = Q^T dl + dO^T P             A = transposed reads of the Q / dO rows,
//                                     B = transposed reads of dl / P
// and each key's 128 gradient values go to its slot position.
template <bool SPARSE, int HPW>
__global__ __launch_bounds__(kBwdThreads, HPW == 1 ? 2 : 1) void k_attn_bwd16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ x_win, const int32_t* __restrict__ win_start, const float* __restrict__ sink,
    const int32_t* __restrict__ q_pos, const float* __restrict__ Dv, const float* __restrict__ lse,
    const uint16_t* __restrict__ dout, int64_t r0, int64_t Tq, int64_t N, int64_t T_win, int k, int window,
    int ratio, float scale, const int32_t* __restrict__ posbuf, int64_t smax, float* __restrict__ G,
    uint16_t* __restrict__ dq, float* __restrict__ dsink_part) {
  constexpr int H = 64 * HPW;
  constexpr float kLog2e = 1.4426950408889634f;
  // Key tiles (a 2-slot ring filled by asynchronous gathers) and the Q / dO
  // rows: rows of 256 B, 16-byte chunk c of row x at position c ^ (x & 15).
  // P and dl: rows (heads) of 64 keys, 8-byte unit u of row x at
  // u ^ pdl_swz(x & 15); with 64 heads they take the key slot of their tile
  // once its keys are consumed (16 KB), so two blocks fit a compute unit.
  __shared__ __align__(16) uint16_t ring[2][kKT * kD];
  __shared__ __align__(16) uint16_t qt[H * kD];
  __shared__ __align__(16) uint16_t ot[H * kD];
  __shared__ __align__(16) uint16_t pdl_sep[HPW == 1 ? 8 : 2 * H * kKT];
  __shared__ __align__(4) uint8_t kval[2][kKT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, col = lane & 15;
  const TileLanes tl(lane, 15);
  const int64_t r = r0 + blockIdx.x;
  const BwdRow w = bwd_row<SPARSE>(r, Tq, N, T_win, k, window, ratio, win_start, q_pos);
  const int64_t nk = w.n_sel + w.n_win;
  const int h0 = wv * 16 * HPW;

  // Q and dO rows (one per head) by asynchronous gathers, laid out like key
  // tiles: instruction i of wave wv fills rows (4 i + wv) 4 .. + 3, lane
  // row + lane / 16, chunk position lane % 16 (source chunk (lane % 16) ^ (row % 16)).
#pragma unroll
  for (int i = 0; i < H / 16; ++i) {
    const int hr = (4 * i + wv) * 4 + (lane >> 4);
    const int c = (lane & 15) ^ (hr & 15);
    gather_lds16(q + (r * H + hr) * kD + c * 8, (uint32_t)(uintptr_t)(qt + (4 * i + wv) * 4 * kD));
    gather_lds16(dout + (r * H + hr) * kD + c * 8, (uint32_t)(uintptr_t)(ot + (4 * i + wv) * 4 * kD));
  }

  // Q and dO fragments (B operands of S^T, dP^T), D_h, lse, sink term.
  Frag<uint16_t> qf[HPW][kD / 32], df[HPW][kD / 32];
  float Dh[HPW], lse2[HPW];
  bool live[HPW];
#pragma unroll
  for (int hb = 0; hb < HPW; ++hb) {
    const int64_t hrow = r * H + h0 + 16 * hb + col;
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) {
      qf[hb][ks].load(q + hrow * kD + 32 * ks + 8 * g);
      df[hb][ks].load(dout + hrow * kD + 32 * ks + 8 * g);
    }
    const float acc = Dv[hrow];
    Dh[hb] = acc;
    const float L = lse[hrow];
    live[hb] = L > -INFINITY;
    lse2[hb] = live[hb] ? L * kLog2e : 0.f;
    if (sink && g == 0) dsink_part[hrow] = live[hb] ? -__expf(sink[h0 + 16 * hb + col] - L) * acc : 0.f;
  }
  const float scale2 = scale * kLog2e;

  const uint16_t* kvb = kv + w.b * N * kD;
  const uint16_t* xwb = x_win + w.b * T_win * kD;
  // A key tile's gathers: instruction j of wave wv fills rows 16 j + grow0
  // (grow0 = 4 wv + lane / 16) as above; the selected indices of a thread's
  // rows are loaded a tile ahead of the gathers. Branch-free: every access is
  // valid (the index clamped to the row; a slot without a key reads the
  // query's own row, finite and masked later).
  const int grow0 = 4 * wv + (lane >> 4);
  auto load_idx = [&](int64_t t, int32_t (&e)[4]) {
    if constexpr (SPARSE) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t kk = t * kKT + 16 * j + grow0;
        e[j] = idx[r * k + (kk < k ? kk : (int64_t)k - 1)];
      }
    }
  };
  const uint16_t* dummy = q + r * H * kD;
  auto issue = [&](int64_t t, const int32_t (&e)[4]) {
    const int sl = (int)(t & 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * j + grow0;
      const int64_t kk = t * kKT + row;
      const bool in_sel = kk < w.n_sel;
      const int64_t en = SPARSE ? (int64_t)e[j] : kk;
      const bool ok_sel = in_sel && en >= 0 && en < N;
      const bool ok_win = !in_sel && kk < nk;
      const int64_t wr = w.lo + (kk - w.n_sel) - w.w0;
      const uint16_t* src = ok_sel ? kvb + en * kD : (ok_win ? xwb + wr * kD : dummy);
      gather_lds16(src + (((lane & 15) ^ (row & 15)) * 8), (uint32_t)(uintptr_t)(ring[sl] + (4 * j + wv) * 4 * kD));
      if ((lane & 15) == 0) kval[sl][row] = (ok_sel || ok_win) ? 1 : 0;
    }
  };

  f32x4 dQ[HPW][kD / 16];
#pragma unroll
  for (int hb = 0; hb < HPW; ++hb)
#pragma unroll
    for (int db = 0; db < kD / 16; ++db) dQ[hb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint32_t qtb = (uint32_t)(uintptr_t)qt, otb = (uint32_t)(uintptr_t)ot;
  const int64_t ntiles = cdiv(nk, kKT);
  const int32_t* prow = posbuf + (r - r0) * smax;
  uint32_t ga[2], gb[4];   // tile-invariant offsets of the key-row gradient product
  gt_offsets(tl, wv, g, col, ga, gb);
  int32_t e_next[4];
  {
    int32_t e0[4];
    load_idx(0, e0);
    if (ntiles > 0) issue(0, e0);
    load_idx(1, e_next);
  }
  for (int64_t t = 0; t < ntiles; ++t) {
    const int sl = (int)(t & 1);
    // Tile t's gathers are complete. The vector memory operations issued after
    // them (index and position loads, gradient-row stores) are the compiler's,
    // and how many of them precede this point depends on its code placement,
    // so the wait does not count them: it drains every outstanding operation
    // (measured cost about 1% of the kernel). The barrier then also means
    // every wave is past the previous tile's use of the other slot.
    wait_vm<0>();
    __syncthreads();
    if (t + 1 < ntiles) {
      issue(t + 1, e_next);
      load_idx(t + 2, e_next);
    }
    const uint32_t tb = (uint32_t)(uintptr_t)ring[sl];
    int32_t pv[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int64_t kk = t * kKT + 16 * nb + col;
      if constexpr (SPARSE) {
        const int32_t v = prow[kk < nk ? kk : nk - 1];
        pv[nb] = kk < nk ? v : -1;
      } else {   // dense rows list window slots only
        const bool win = kk >= w.n_sel && kk < nk;
        const int32_t v = prow[win ? kk - w.n_sel : 0];
        pv[nb] = win ? v : -1;
      }
    }

    // ---- S^T = K Q^T and dP^T = K dO^T (keys 16 kb + 4 g + rr, head column col)
    float s[HPW][4][4], dp[HPW][4][4];
    {
      f32x4 as[4][HPW], ad[4][HPW];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) {
          as[kb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
          ad[kb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int ks = 0; ks < kD / 32; ++ks) {
        uint32_t ka = (((uint32_t)(64 * ks)) ^ tl.kx) + (tb + tl.kofs);
        opaque(ka);
        Frag<uint16_t> a[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) a[kb].v = lds_read_b128(ka + 4096 * kb);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int hb = 0; hb < HPW; ++hb) {
            as[kb][hb] = mma8(a[kb], qf[hb][ks], as[kb][hb]);
            ad[kb][hb] = mma8(a[kb], df[hb][ks], ad[kb][hb]);
          }
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
          for (int hb = 0; hb < HPW; ++hb) {
            s[hb][kb][rr] = as[kb][hb][rr];
            dp[hb][kb][rr] = ad[kb][hb][rr];
          }
    }
    // ---- P = exp(l - lse), scale * dl = scale * P (dP - D); no key or no
    // softmax mass: 0
    {
      uint32_t okw[4];    // byte rr of word kb: key 16 kb + 4 g + rr holds a key
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) okw[kb] = reinterpret_cast<const uint32_t*>(kval[sl])[4 * kb + g];
#pragma unroll
      for (int hb = 0; hb < HPW; ++hb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const bool ok = live[hb] && ((okw[kb] >> (8 * rr)) & 1u);
            const float pv = ok ? __builtin_amdgcn_exp2f(fmaf(s[hb][kb][rr], scale2, -lse2[hb])) : 0.f;
            s[hb][kb][rr] = pv;
            dp[hb][kb][rr] = scale * pv * (dp[hb][kb][rr] - Dh[hb]);
          }
    }
    // ---- dQ^T += K^T (scale dl)^T (K-slot order of the transposed reads)
    {
      uint32_t va[kD / 16];
#pragma unroll
      for (int db = 0; db < kD / 16; ++db) {
        va[db] = (((uint32_t)(32 * db)) ^ tl.vx) + (tb + tl.vofs);
        opaque(va[db]);
      }
#pragma unroll
      for (int grp = 0; grp < 2; ++grp) {
        Frag<uint16_t> lf[HPW];
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) {
          lf[hb].v[0] = (int)cvt_pk_bf16(dp[hb][2 * grp][0], dp[hb][2 * grp][1]);
          lf[hb].v[1] = (int)cvt_pk_bf16(dp[hb][2 * grp][2], dp[hb][2 * grp][3]);
          lf[hb].v[2] = (int)cvt_pk_bf16(dp[hb][2 * grp + 1][0], dp[hb][2 * grp + 1][1]);
          lf[hb].v[3] = (int)cvt_pk_bf16(dp[hb][2 * grp + 1][2], dp[hb][2 * grp + 1][3]);
        }
#pragma unroll
        for (int db = 0; db < kD / 16; ++db) {
          const s16x4 lo4 = lds_read_tr16(va[db] + 8192 * grp);
          const s16x4 hi4 = lds_read_tr16(va[db] + 8192 * grp + 4096);
          const i32x2 l2 = __builtin_bit_cast(i32x2, lo4), h2 = __builtin_bit_cast(i32x2, hi4);
          Frag<uint16_t> vf;
          vf.v = i32x4{l2[0], l2[1], h2[0], h2[1]};
#pragma unroll
          for (int hb = 0; hb < HPW; ++hb) dQ[hb][db] = mma8(vf, lf[hb], dQ[hb][db]);
        }
      }
    }
    // ---- key-row gradients of the tile (dense layers: only tiles holding
    // window keys; the entries' gradients come from k_attn_bwd_dense_kv)
    if (SPARSE || t * kKT + kKT > w.n_sel) {   // block-uniform
      // P and scale * dl to LDS, [head][key] (64 heads: into this tile's key
      // slot, once every wave is done with its keys)
      if constexpr (HPW == 1) __syncthreads();
      const uint32_t plb = HPW == 1 ? tb : (uint32_t)(uintptr_t)pdl_sep;
      const uint32_t dlb = plb + (uint32_t)(H * kKT * 2);
      write_pdl<HPW>(plb, dlb, h0, g, col, s, dp);
      __syncthreads();
      f32x4 acc[2][4];
#pragma unroll
      for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[d2][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      gt_accum<H>(acc, qtb, otb, plb, dlb, ga, gb);
      // lane: rows d = 16 db + 4 g .. + 3 of key 16 nb + col
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        if (pv[nb] < 0) continue;
        float* gr = G + (int64_t)pv[nb] * kD;
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2) {
          const int db = 2 * wv + d2;
          *reinterpret_cast<float4*>(gr + 16 * db + 4 * g) =
              make_float4(acc[d2][nb][0], acc[d2][nb][1], acc[d2][nb][2], acc[d2][nb][3]);
        }
      }
    }
  }
  // ---- dq: lane holds d = 16 db + 4 g .. + 3 of head h0 + 16 hb + col
#pragma unroll
  for (int hb = 0; hb < HPW; ++hb) {
    uint16_t* dqr = dq + (r * H + h0 + 16 * hb + col) * kD;
#pragma unroll
    for (int db = 0; db < kD / 16; ++db)
      *reinterpret_cast<uint2*>(dqr + 16 * db + 4 * g) =
          make_uint2(cvt_pk_bf16(dQ[hb][db][0], dQ[hb][db][1]), cvt_pk_bf16(dQ[hb][db][2], dQ[hb][db][3]));
  }
}

// Dense layers, compressed entries: one block per (block of 64 entries,
// sequence, segment of query rows). The entries stay in LDS; for every query
// row of the segment that sees at least one of them, the block gathers the
// row's Q and dO, forms S^T, dP^T, P and scale * dl for the 64 entries
// (entries past n(p) get P = 0) and adds G^T = Q^T (scale dl) + dO^T P to
// accumulators that live in registers across the rows. Each block writes its
// segment's partial once; k_bwd_seg_reduce adds the segments in order. This
// replaces a 512-byte contribution row per (query, entry). Block order:
// consecutive block numbers go round-robin to the 8 XCDs, and all entry
// blocks of one segment get numbers of one residue mod 8, so they run on one
// XCD and each row's Q and dO come from that XCD's L2 after the first read
// (rather than from HBM once per XCD that holds one of the entry blocks).
template <int HPW>
__global__ __launch_bounds__(kBwdThreads, HPW == 1 ? 2 : 1) void k_attn_bwd_dense_kv(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ q_pos,
    const float* __restrict__ Dv, const float* __restrict__ lse, const uint16_t* __restrict__ dout, int64_t Tq,
    int64_t N, int ratio, float scale, int64_t seg, int nseg, int64_t nsg, int nkb, float* __restrict__ part) {
  constexpr int H = 64 * HPW;
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ __align__(16) uint16_t kt[kKT * kD];      // the block's 64 entries
  __shared__ __align__(16) uint16_t qt[H * kD];        // the current row's Q (one row per head)
  __shared__ __align__(16) uint16_t ot[H * kD];        // and dO
  __shared__ __align__(16) uint16_t pdl[2 * H * kKT];  // P, then scale * dl, [head][key]
  __shared__ int nvis[kBwdThreads];                      // n(p) of the next 256 rows of the segment

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, col = lane & 15;
  const TileLanes tl(lane, 15);
  const int64_t xcd = blockIdx.x % 8, kx = blockIdx.x / 8;
  const int64_t sg = (kx / nkb) * 8 + xcd;   // segment b * nseg + sgi
  if (sg >= nsg) return;                      // uniform: the grid is padded to whole groups of 8
  const int64_t e0 = (kx % nkb) * kKT;
  const int64_t b = sg / nseg, sgi = sg % nseg;
  const int64_t t0 = sgi * seg, t1 = (t0 + seg) < Tq ? (t0 + seg) : Tq;
  const int h0 = wv * 16 * HPW;
  const float scale2 = scale * kLog2e;
  // the block's entries (rows past N read entry N - 1: never visible)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 16 * j + 4 * wv + (lane >> 4);
    const int64_t e = (e0 + row) < N ? (e0 + row) : N - 1;
    gather_lds16(kv + (b * N + e) * kD + (((lane & 15) ^ (row & 15)) * 8),
                 (uint32_t)(uintptr_t)(kt + (4 * j + wv) * 4 * kD));
  }
  const uint32_t tb = (uint32_t)(uintptr_t)kt, qtb = (uint32_t)(uintptr_t)qt, otb = (uint32_t)(uintptr_t)ot;
  const uint32_t plb = (uint32_t)(uintptr_t)pdl, dlb = plb + (uint32_t)(H * kKT * 2);
  uint32_t ga[2], gb[4];
  gt_offsets(tl, wv, g, col, ga, gb);
  f32x4 acc[2][4];
#pragma unroll
  for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[d2][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t t = t0; t < t1; ++t) {
    const int64_t r = b * Tq + t;
    if (((t - t0) & (kBwdThreads - 1)) == 0) {   // uniform: stage n(p) of the next 256 rows
      __syncthreads();
      const int64_t tt = t + tid;
      nvis[tid] = tt < t1 ? (int)visible(q_pos[b * Tq + tt], ratio, N) : 0;
      __syncthreads();
    }
    const int n = __builtin_amdgcn_readfirstlane(nvis[(t - t0) & (kBwdThreads - 1)]);
    if (n <= e0) continue;   // uniform: none of the block's entries is visible
    // the row's Q and dO rows, laid out like key tiles
#pragma unroll
    for (int i = 0; i < H / 16; ++i) {
      const int hr = (4 * i + wv) * 4 + (lane >> 4);
      const int c = (lane & 15) ^ (hr & 15);
      gather_lds16(q + (r * H + hr) * kD + c * 8, (uint32_t)(uintptr_t)(qt + (4 * i + wv) * 4 * kD));
      gather_lds16(dout + (r * H + hr) * kD + c * 8, (uint32_t)(uintptr_t)(ot + (4 * i + wv) * 4 * kD));
    }
    float Dh[HPW], lse2[HPW];
    bool live[HPW];
#pragma unroll
    for (int hb = 0; hb < HPW; ++hb) {
      const int64_t hrow = r * H + h0 + 16 * hb + col;
      Dh[hb] = Dv[hrow];
      const float L = lse[hrow];
      live[hb] = L > -INFINITY;
      lse2[hb] = live[hb] ? L * kLog2e : 0.f;
    }
    wait_vm<0>();
    __syncthreads();
    // S^T = K Q^T, dP^T = K dO^T (entries 16 kb + 4 g + rr, head column col);
    // the B operands come from the Q / dO rows in LDS
    float sv[HPW][4][4], dp[HPW][4][4];
    {
      f32x4 as[4][HPW], ad[4][HPW];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) {
          as[kb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
          ad[kb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int ks = 0; ks < kD / 32; ++ks) {
        uint32_t ka = (((uint32_t)(64 * ks)) ^ tl.kx) + tl.kofs;
        opaque(ka);
        Frag<uint16_t> a[4], qf[HPW], df[HPW];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) a[kb].v = lds_read_b128(tb + ka + 4096 * kb);
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) {
          qf[hb].v = lds_read_b128(qtb + ka + 4096 * (wv * HPW + hb));
          df[hb].v = lds_read_b128(otb + ka + 4096 * (wv * HPW + hb));
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int hb = 0; hb < HPW; ++hb) {
            as[kb][hb] = mma8(a[kb], qf[hb], as[kb][hb]);
            ad[kb][hb] = mma8(a[kb], df[hb], ad[kb][hb]);
          }
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
          for (int hb = 0; hb < HPW; ++hb) {
            const bool ok = live[hb] && (e0 + 16 * kb + 4 * g + rr) < n;
            const float pv = ok ? __builtin_amdgcn_exp2f(fmaf(as[kb][hb][rr], scale2, -lse2[hb])) : 0.f;
            sv[hb][kb][rr] = pv;
            dp[hb][kb][rr] = scale * pv * (ad[kb][hb][rr] - Dh[hb]);
          }
    }
    write_pdl<HPW>(plb, dlb, h0, g, col, sv, dp);
    __syncthreads();
    gt_accum<H>(acc, qtb, otb, plb, dlb, ga, gb);
    __syncthreads();   // the next row's gathers and P / dl writes reuse qt, ot, pdl
  }
  // partial of this segment: lane rows d = 16 db + 4 g .. + 3 of entry e0 + 16 nb + col
  float* pb = part + ((b * nseg + sgi) * N + e0) * kD;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    if (e0 + 16 * nb + col >= N) continue;
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2) {
      const int db = 2 * wv + d2;
      *reinterpret_cast<float4*>(pb + (16 * nb + col) * kD + 16 * db + 4 * g) =
          make_float4(acc[d2][nb][0], acc[d2][nb][1], acc[d2][nb][2], acc[d2][nb][3]);
    }
  }
}

// dkv[b, e] = sum over segments s (in order) of part[b, s, e]: one wave per entry.
__global__ __launch_bounds__(kBwdThreads) void k_bwd_seg_reduce(const float* __restrict__ part, int64_t B, int64_t N,
                                                                int nseg, float* __restrict__ dkv) {
  const int64_t i = (int64_t)blockIdx.x * (kBwdThreads / 64) + (threadIdx.x >> 6);
  if (i >= B * N) return;
  const int lane = threadIdx.x & 63;
  const int64_t b = i / N, e = i % N;
  float2 acc = make_float2(0.f, 0.f);
  for (int sg = 0; sg < nseg; ++sg) {
    const float2 v = *reinterpret_cast<const float2*>(part + ((b * nseg + sg) * N + e) * kD + 2 * lane);
    acc.x += v.x;
    acc.y += v.y;
  }
  *reinterpret_cast<float2*>(dkv + i * kD + 2 * lane) = acc;
}

// One block per key: wave w sums the w-th quarter of the key's contribution
// list (8 loads in flight, added in list order), then the quarters are added
// in order to the previous passes' sum (when `accumulate`). The split
// depends only on the list length, so the result is the same on every run.
__global__ __launch_bounds__(kBwdThreads) void k_bwd_reduce(const float* __restrict__ G,
                                                            const uint32_t* __restrict__ off, int64_t nids,
                                                            int64_t N, int64_t T_win, float* __restrict__ dkv,
                                                            float* __restrict__ dx_win, int accumulate, int win_only) {
  __shared__ float2 part[kBwdThreads / 64][64];
  const int64_t id = blockIdx.x;   // win_only (dense layers): ids are window rows b T_win + t
  if (id >= nids) return;          // uniform: the grid has one block per id
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t u0 = off[id], len = off[id + 1] - u0;
  const uint32_t a = u0 + (uint32_t)(((uint64_t)len * wv) / 4), e = u0 + (uint32_t)(((uint64_t)len * (wv + 1)) / 4);
  const float* gp = G + 2 * lane;
  float2 acc = make_float2(0.f, 0.f);
  uint32_t u = a;
  for (; u + 8 <= e; u += 8) {
    float2 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const float2*>(gp + (int64_t)(u + i) * kD);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc.x += v[i].x;
      acc.y += v[i].y;
    }
  }
  for (; u < e; ++u) {
    const float2 v = *reinterpret_cast<const float2*>(gp + (int64_t)u * kD);
    acc.x += v.x;
    acc.y += v.y;
  }
  part[wv][lane] = acc;
  __syncthreads();
  if (wv == 0) {
    const int64_t b = id / (N + T_win), j = id % (N + T_win);
    float* o = (win_only ? dx_win + id * kD : j < N ? dkv + (b * N + j) * kD : dx_win + (b * T_win + (j - N)) * kD) +
               2 * lane;
    float2 t = accumulate ? *reinterpret_cast<const float2*>(o) : make_float2(0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kBwdThreads / 64; ++w) {
      t.x += part[w][lane].x;
      t.y += part[w][lane].y;
    }
    *reinterpret_cast<float2*>(o) = t;
  }
}

// Sink gradient, first level: block j sums rows [j R, (j + 1) R) for every
// head (thread: head tid % H, rows tid / H + (256 / H) i), the row groups
// added in order; part[j][h].
__global__ __launch_bounds__(kBwdThreads) void k_bwd_sink_part(const float* __restrict__ rowv, int64_t rows, int H,
                                                               int64_t R, float* __restrict__ part) {
  __shared__ float red[kBwdThreads];
  const int tid = threadIdx.x, h = tid % H, rg = tid / H, ng = kBwdThreads / H;
  const int64_t r0 = (int64_t)blockIdx.x * R;
  const int64_t r1 = r0 + R < rows ? r0 + R : rows;
  float s = 0.f;
  for (int64_t r = r0 + rg; r < r1; r += ng) s += rowv[r * H + h];
  red[tid] = s;
  __syncthreads();
  if (rg == 0) {
    float t = 0.f;
    for (int gi = 0; gi < ng; ++gi) t += red[gi * H + h];
    part[(int64_t)blockIdx.x * H + h] = t;
  }
}

// Second level: dsink[h] = sum over blocks j of part[j][h], in order.
__global__ __launch_bounds__(kBwdThreads) void k_bwd_sink_final(const float* __restrict__ part, int nb, int H,
                                                                float* __restrict__ dsink) {
  const int h = threadIdx.x;
  if (h >= H) return;
  float t = 0.f;
  for (int j = 0; j < nb; ++j) t += part[(int64_t)j * H + h];
  dsink[h] = t;
}

// ------------------------------------------------------------------ host side

struct BwdPlan {
  int64_t rows, smax, rows_pass, nchunks, nids, nscan, nkb, seg, nseg;
  size_t o_cnt, o_total, o_off, o_bsum, o_pos, o_g, o_sink, o_spart, o_delta, o_part, bytes;
};

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

static BwdPlan bwd_plan(bool sparse, int64_t B, int64_t Tq, int64_t N, int64_t T_win, int H, int k, int window) {
  BwdPlan p;
  p.rows = B * Tq;
  const int64_t wmax = window < T_win ? (int64_t)window : T_win;
  // contribution slots per query row: selected entries and window rows
  // (sparse), window rows only (dense)
  p.smax = (sparse ? (int64_t)k : 0) + wmax;
  if (p.smax < 1) p.smax = 1;
  int64_t rp = kBwdGBudget / (p.smax * kD * 4) / kBwdQc * kBwdQc;
  if (rp < kBwdQc) rp = kBwdQc;
  p.rows_pass = rp < p.rows ? rp : p.rows;
  p.nchunks = cdiv(p.rows_pass, kBwdQc);
  p.nids = sparse ? B * (N + T_win) : B * T_win;
  p.nscan = cdiv(p.nids, kScanBlock);
  // dense entries: blocks of 64 entries x sequences x segments of query rows,
  // about 2048 blocks
  p.nkb = cdiv(N, kKT);
  p.seg = 1;
  p.nseg = 0;
  if (!sparse && N > 0) {
    int64_t ns = cdiv(2048, p.nkb * B);
    if (ns > Tq) ns = Tq;
    if (ns < 1) ns = 1;
    p.seg = cdiv(Tq, ns);
    p.nseg = cdiv(Tq, p.seg);
  }
  size_t o = 0;
  p.o_cnt = o;   o += align256((size_t)p.nchunks * p.nids * 4);
  p.o_total = o; o += align256((size_t)p.nids * 4);
  p.o_off = o;   o += align256((size_t)(p.nids + 1) * 4);
  p.o_bsum = o;  o += align256((size_t)p.nscan * 4);
  p.o_pos = o;   o += align256((size_t)p.rows_pass * p.smax * 4);
  p.o_g = o;     o += align256((size_t)p.rows_pass * p.smax * kD * 4);
  p.o_sink = o;  o += align256((size_t)p.rows * H * 4);
  p.o_spart = o; o += align256((size_t)kSinkBlocks * H * 4);
  p.o_delta = o; o += align256((size_t)p.rows * H * 4);
  p.o_part = o;  o += align256((size_t)B * p.nseg * N * kD * 4);
  p.bytes = o;
  return p;
}

size_t attn_bwd_ws_bytes(bool sparse, int64_t B, int64_t Tq, int64_t N, int64_t T_win, int H, int k, int window) {
  if (B <= 0 || Tq <= 0) return 0;
  return bwd_plan(sparse, B, Tq, N, T_win, H, k, window).bytes;
}

static unsigned fill_grid(int64_t n) {
  const int64_t b = cdiv(n, kBwdThreads);
  return (unsigned)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

template <bool SPARSE>
static hipError_t run_attn_bwd(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const uint16_t* x_win,
                               const int32_t* win_start, const float* sink, const int32_t* q_pos,
                               const uint16_t* out, const float* lse, const uint16_t* dout, int64_t B, int64_t Tq,
                               int64_t N, int64_t T_win, int H, int k, int window, int ratio, float scale,
                               uint16_t* dq, float* dkv, float* dx_win, float* dsink, void* ws, hipStream_t s) {
  const BwdPlan p = bwd_plan(SPARSE, B, Tq, N, T_win, H, k, window);
  uint8_t* wb = static_cast<uint8_t*>(ws);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(wb + p.o_cnt);
  uint32_t* total = reinterpret_cast<uint32_t*>(wb + p.o_total);
  uint32_t* off = reinterpret_cast<uint32_t*>(wb + p.o_off);
  uint32_t* bsum = reinterpret_cast<uint32_t*>(wb + p.o_bsum);
  int32_t* pos = reinterpret_cast<int32_t*>(wb + p.o_pos);
  float* G = reinterpret_cast<float*>(wb + p.o_g);
  float* spart = reinterpret_cast<float*>(wb + p.o_sink);
  float* delta = reinterpret_cast<float*>(wb + p.o_delta);
  k_bwd_delta<<<(unsigned)cdiv(p.rows * H, kBwdThreads / 16), kBwdThreads, 0, s>>>(out, dout, p.rows * H, delta);
  for (int64_t r0 = 0; r0 < p.rows; r0 += p.rows_pass) {
    const int64_t r1 = r0 + p.rows_pass < p.rows ? r0 + p.rows_pass : p.rows;
    const int64_t nr = r1 - r0;
    const int64_t nch = cdiv(nr, kBwdQc);
    if (p.nids > 0) {   // keys that take contributions (none: a dense layer without window rows)
      k_fill_u32<<<fill_grid(nch * p.nids), kBwdThreads, 0, s>>>(cnt, nch * p.nids, 0u);
      k_bwd_count<SPARSE><<<(unsigned)nr, kBwdThreads, 0, s>>>(idx, win_start, q_pos, r0, Tq, N, T_win, k, window,
                                                               ratio, p.nids, cnt);
      k_bwd_chunk_scan<<<(unsigned)cdiv(p.nids, kBwdThreads), kBwdThreads, 0, s>>>(cnt, p.nids, (int)nch, total);
      k_bwd_scan_sums<<<(unsigned)p.nscan, kBwdThreads, 0, s>>>(total, p.nids, bsum);
      k_bwd_scan_top<<<1, kBwdThreads, 0, s>>>(bsum, p.nscan);
      k_bwd_scan_apply<<<(unsigned)p.nscan, kBwdThreads, 0, s>>>(total, p.nids, bsum, off);
      k_bwd_place<SPARSE><<<(unsigned)nch, kBwdThreads, 0, s>>>(idx, win_start, q_pos, r0, r1, Tq, N, T_win, k,
                                                                window, ratio, p.nids, cnt, off, pos, p.smax);
    }
    timer_before(CSA_KID_ATTN_BWD, s);
    if (H == 64)
      k_attn_bwd16<SPARSE, 1><<<(unsigned)nr, kBwdThreads, 0, s>>>(q, kv, idx, x_win, win_start, sink, q_pos, delta,
                                                                  lse, dout, r0, Tq, N, T_win, k, window, ratio,
                                                                  scale, pos, p.smax, G, dq, spart);
    else
      k_attn_bwd16<SPARSE, 2><<<(unsigned)nr, kBwdThreads, 0, s>>>(q, kv, idx, x_win, win_start, sink, q_pos, delta,
                                                                  lse, dout, r0, Tq, N, T_win, k, window, ratio,
                                                                  scale, pos, p.smax, G, dq, spart);
    hipError_t e = hipGetLastError();
    timer_after(CSA_KID_ATTN_BWD, s);
    if (e != hipSuccess) return e;
    if (p.nids > 0)
      k_bwd_reduce<<<(unsigned)p.nids, kBwdThreads, 0, s>>>(G, off, p.nids, N, T_win, dkv, dx_win, r0 > 0 ? 1 : 0,
                                                            SPARSE ? 0 : 1);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!SPARSE && p.nseg > 0) {   // dense: the entries' gradients, summed over query segments
    float* part = reinterpret_cast<float*>(wb + p.o_part);
    const int64_t nsg = B * p.nseg;
    const unsigned grid = (unsigned)(p.nkb * 8 * cdiv(nsg, 8));
    timer_before(CSA_KID_ATTN_BWD, s);
    if (H == 64)
      k_attn_bwd_dense_kv<1><<<grid, kBwdThreads, 0, s>>>(q, kv, q_pos, delta, lse, dout, Tq, N, ratio, scale, p.seg,
                                                         (int)p.nseg, nsg, (int)p.nkb, part);
    else
      k_attn_bwd_dense_kv<2><<<grid, kBwdThreads, 0, s>>>(q, kv, q_pos, delta, lse, dout, Tq, N, ratio, scale, p.seg,
                                                         (int)p.nseg, nsg, (int)p.nkb, part);
    hipError_t e = hipGetLastError();
    timer_after(CSA_KID_ATTN_BWD, s);
    if (e != hipSuccess) return e;
    k_bwd_seg_reduce<<<(unsigned)cdiv(B * N, kBwdThreads / 64), kBwdThreads, 0, s>>>(part, B, N, (int)p.nseg, dkv);
  }
  if (sink && dsink) {
    float* sp2 = reinterpret_cast<float*>(wb + p.o_spart);
    const int64_t R = cdiv(p.rows, kSinkBlocks);
    const int nb = (int)cdiv(p.rows, R);
    k_bwd_sink_part<<<(unsigned)nb, kBwdThreads, 0, s>>>(spart, p.rows, H, R, sp2);
    k_bwd_sink_final<<<1, kBwdThreads, 0, s>>>(sp2, nb, H, dsink);
  }
  return hipGetLastError();
}

hipError_t launch_attn_bwd(bool sparse, const void* q, const void* kv, const int32_t* idx, const void* x_win,
                           const int32_t* win_start, const float* sink, const int32_t* q_pos, const void* out,
                           const float* lse, const void* dout, int64_t B, int64_t Tq, int64_t N, int64_t T_win,
                           int H, int k, int window, int ratio, float scale, void* dq, float* dkv, float* dx_win,
                           float* dsink, void* ws, hipStream_t s) {
  if (B * Tq == 0) return hipSuccess;
  auto bf = [](const void* p) { return static_cast<const uint16_t*>(p); };
  if (sparse)
    return run_attn_bwd<true>(bf(q), bf(kv), idx, bf(x_win), win_start, sink, q_pos, bf(out), lse, bf(dout), B, Tq,
                              N, T_win, H, k, window, ratio, scale, static_cast<uint16_t*>(dq), dkv, dx_win, dsink,
                              ws, s);
  return run_attn_bwd<false>(bf(q), bf(kv), idx, bf(x_win), win_start, sink, q_pos, bf(out), lse, bf(dout), B, Tq,
                             N, T_win, H, k, window, ratio, scale, static_cast<uint16_t*>(dq), dkv, dx_win, dsink,
                             ws, s);
}

}  // namespace csa
