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
//   online softmax   per head = per lane column; the sink is one more logit
//                    (sink_h, value 0): the float32 kernel starts its running
//                    max and denominator from it, the bf16 kernel adds it
//                    after its last tile,
//   O^T += V^T P^T   MFMA, P^T straight from the S^T accumulators: the 8
//                    K-slots of a lane are the 2x4 keys it already holds, and
//                    V^T is read from LDS with the same key permutation.
// bf16: v_mfma_f32_16x16x32_bf16; f32: v_mfma_f32_16x16x4_f32 (8 per 32 keys).
// With few queries (decode) the key list is split across blocks (a fixed
// count from the shapes, never from timing) and the partial (O, max, sum)
// triples are merged in a fixed order, so results are deterministic.
#include "attn_tile.hpp"

namespace csa {

template <typename T> struct AttnTypes;
template <> struct AttnTypes<uint16_t> {
  static constexpr int KP = kD + 8;     // row pitch of the row-major tile (elements)
};
template <> struct AttnTypes<float> {
  static constexpr int KP = kD + 4;
};

// Position of key `key` of value-row d in the transposed tile. Groups of 4
// consecutive keys stay together; the group index is XOR-swizzled by a
// function of d so that both the packed 4-key stores of the gather and the
// 4-key fragment loads of the P*V product spread over all LDS banks.
__device__ __forceinline__ int vt_pos(int d, int key) {
  const int h = (d & 15) ^ ((d >> 3) & 15);
  return d * kKT + (key ^ (4 * h));
}

// Store element e of four consecutive key rows (f[0..3]) as 4 packed keys.
__device__ __forceinline__ void store_vt4(uint16_t* p, const Frag<uint16_t>* f, int e) {
  *reinterpret_cast<uint2*>(p) = make_uint2(f[0].elem(e) | (f[1].elem(e) << 16), f[2].elem(e) | (f[3].elem(e) << 16));
}
__device__ __forceinline__ void store_vt4(float* p, const Frag<float>* f, int e) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0].elem(e), f[1].elem(e), f[2].elem(e), f[3].elem(e));
}

// One block: one query row, NW waves x HPW blocks of 16 heads, one key split.
template <typename T, bool SPARSE, int NW, int HPW>
__global__ __launch_bounds__(NW * 64) void k_attn(
    const T* __restrict__ q, const T* __restrict__ kv, const int32_t* __restrict__ idx, const T* __restrict__ x_win,
    const int32_t* __restrict__ win_start, const float* __restrict__ sink, const int32_t* __restrict__ q_pos,
    int64_t Tq, int64_t N, int64_t T_win, int wring, int H, int k, int window, int ratio, float scale, int S,
    T* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int KP = AttnTypes<T>::KP;
  constexpr int NT = NW * 64;
  constexpr int PAIRS = 256 / NT;            // (4-row quad, 16-byte column) pairs per thread per tile
  constexpr int TPS = (sizeof(T) == 2 ? 2 : 1) * (NT >= 128 ? 1 : 1);   // tiles per super-tile
  constexpr int SUPER = TPS * kKT;
  __shared__ __align__(16) T Kt[kKT * KP];
  __shared__ __align__(16) T Vt[kD * kKT];
  __shared__ int valid[kKT];
  __shared__ int sidx[SUPER];

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
  // row of window position lo: lo - w0, or lo mod T_win for a ring (a window
  // of at most T_win rows wraps at most once)
  const int64_t wrow0 = wring ? lo % (T_win > 0 ? T_win : 1) : lo - w0;

  // heads of this lane: h0 + 16 * hb + col
  const int h0 = hg * (NW * 16 * HPW) + wv * 16 * HPW;
  Frag<T> qf[HPW][kD / 32];
#pragma unroll
  for (int hb = 0; hb < HPW; ++hb) {
    const T* qrow = q + (r * H + h0 + 16 * hb + col) * kD;
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) qf[hb][ks].load(qrow + 32 * ks + 8 * g);
  }
  const bool has_sink = (sink != nullptr) && sp == 0;
  float m[HPW], lsum[HPW];
  f32x4 O[HPW][kD / 16];
#pragma unroll
  for (int hb = 0; hb < HPW; ++hb) {
    m[hb] = has_sink ? sink[h0 + 16 * hb + col] : -INFINITY;
    lsum[hb] = (has_sink && g == 0) ? 1.f : 0.f;
#pragma unroll
    for (int db = 0; db < kD / 16; ++db) O[hb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Keys are walked in super-tiles: every gather of a super-tile is issued
  // before its first tile is computed (one round of memory latency per
  // super-tile). A thread gathers, per tile, PAIRS quads of 4 consecutive key
  // rows at one 16-byte column, so it can store V^T as packed 4-key groups.
  for (int64_t s0 = kbeg; s0 < kend; s0 += SUPER) {
    const int ns = (int)((kend - s0) < SUPER ? (kend - s0) : SUPER);
    if (SPARSE) {
      for (int i = tid; i < SUPER; i += NT) {
        const int64_t ki = s0 + i;
        sidx[i] = (i < ns && ki < n_sel) ? idx[r * k + ki] : -1;
      }
      __syncthreads();
    }
    Frag<T> buf[TPS][PAIRS][4];
    bool okb[TPS][PAIRS][4];
#pragma unroll
    for (int tt = 0; tt < TPS; ++tt)
#pragma unroll
      for (int pp = 0; pp < PAIRS; ++pp) {
        const int pr = tid + pp * NT;
        const int mq = pr >> 4, cc = pr & 15;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kr = tt * kKT + 4 * mq + i;        // key within the super-tile
          const int64_t ki = s0 + kr;
          const T* src = nullptr;
          if (kr < ns) {
            if (ki < n_sel) {
              const int64_t e = SPARSE ? (int64_t)sidx[kr] : ki;
              if (e >= 0 && e < N) src = kv + (b * N + e) * kD;
            } else {
              int64_t wr = wrow0 + (ki - n_sel);
              if (wr >= T_win) wr -= T_win;
              src = x_win + (b * T_win + wr) * kD;
            }
          }
          okb[tt][pp][i] = src != nullptr;
          if (src) buf[tt][pp][i].load(src + 8 * cc);
          else buf[tt][pp][i].zero();
        }
      }
#pragma unroll
    for (int tt = 0; tt < TPS; ++tt) {
      if (tt * kKT >= ns) break;
      const int nt = (ns - tt * kKT) < kKT ? (ns - tt * kKT) : kKT;
#pragma unroll
      for (int pp = 0; pp < PAIRS; ++pp) {
        const int pr = tid + pp * NT;
        const int mq = pr >> 4, cc = pr & 15;
#pragma unroll
        for (int i = 0; i < 4; ++i) buf[tt][pp][i].store(&Kt[(4 * mq + i) * KP + 8 * cc]);
#pragma unroll
        for (int e = 0; e < 8; ++e) store_vt4(&Vt[vt_pos(8 * cc + e, 4 * mq)], buf[tt][pp], e);
        if (cc == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) valid[4 * mq + i] = okb[tt][pp][i];
        }
      }
      __syncthreads();

      // ---- S^T = K Q^T for 4 blocks of 16 keys; each K fragment feeds HPW head blocks
      float s[HPW][4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        f32x4 acc[HPW];
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const T* krow = &Kt[(16 * kb + col) * KP + 8 * g];
#pragma unroll
        for (int ks = 0; ks < kD / 32; ++ks) {
          Frag<T> a;
          a.load(krow + 32 * ks);
#pragma unroll
          for (int hb = 0; hb < HPW; ++hb) acc[hb] = mma8(a, qf[hb][ks], acc[hb]);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int key = 16 * kb + 4 * g + rr;
          const bool ok = key < nt && valid[key];
#pragma unroll
          for (int hb = 0; hb < HPW; ++hb) s[hb][kb][rr] = ok ? acc[hb][rr] * scale : -INFINITY;
        }
      }
      // ---- online softmax (per head = per column)
#pragma unroll
      for (int hb = 0; hb < HPW; ++hb) {
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) tmax = fmaxf(tmax, s[hb][kb][rr]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float mnew = fmaxf(m[hb], tmax);
        const bool live = mnew != -INFINITY;
        const float alpha = live ? __expf(m[hb] - mnew) : 1.f;
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const float pv = live ? __expf(s[hb][kb][rr] - mnew) : 0.f;
            s[hb][kb][rr] = pv;
            psum += pv;
          }
        lsum[hb] = fmaf(lsum[hb], alpha, psum);
        m[hb] = mnew;
#pragma unroll
        for (int db = 0; db < kD / 16; ++db) O[hb][db] *= alpha;
      }

      // ---- O^T += V^T P^T, two groups of 32 keys. K-slot t of lane group g is
      // key 4g+t (t < 4) or 16+4g+(t-4) (t >= 4) of the group.
#pragma unroll
      for (int grp = 0; grp < 2; ++grp) {
        Frag<T> pf[HPW];
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) {
          if constexpr (sizeof(T) == 2) {
            pf[hb].v[0] = (int)pack_bf16x2(s[hb][2 * grp][0], s[hb][2 * grp][1]);
            pf[hb].v[1] = (int)pack_bf16x2(s[hb][2 * grp][2], s[hb][2 * grp][3]);
            pf[hb].v[2] = (int)pack_bf16x2(s[hb][2 * grp + 1][0], s[hb][2 * grp + 1][1]);
            pf[hb].v[3] = (int)pack_bf16x2(s[hb][2 * grp + 1][2], s[hb][2 * grp + 1][3]);
          } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) pf[hb].v[t] = s[hb][2 * grp + (t >> 2)][t & 3];
          }
        }
#pragma unroll
        for (int db = 0; db < kD / 16; ++db) {
          const int d = 16 * db + col;
          Frag<T> va;
          va.load_split(&Vt[vt_pos(d, 32 * grp + 4 * g)], &Vt[vt_pos(d, 32 * grp + 16 + 4 * g)]);
#pragma unroll
          for (int hb = 0; hb < HPW; ++hb) O[hb][db] = mma8(va, pf[hb], O[hb][db]);
        }
      }
      __syncthreads();
    }
  }

#pragma unroll
  for (int hb = 0; hb < HPW; ++hb) {
    float l = lsum[hb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int head = h0 + 16 * hb + col;
    if (S == 1) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      T* orow = out + (r * H + head) * kD;
#pragma unroll
      for (int db = 0; db < kD / 16; ++db) {
        const float v[4] = {O[hb][db][0] * inv, O[hb][db][1] * inv, O[hb][db][2] * inv, O[hb][db][3] * inv};
        Elem<T>::store4(orow + 16 * db + 4 * g, v);
      }
      if (lse && g == 0) lse[r * H + head] = l > 0.f ? m[hb] + __logf(l) : -INFINITY;
    } else {
      const int64_t pi = (r * H + head) * S + sp;
      float* po = part_o + pi * kD;
#pragma unroll
      for (int db = 0; db < kD / 16; ++db)
        *reinterpret_cast<float4*>(po + 16 * db + 4 * g) = make_float4(O[hb][db][0], O[hb][db][1], O[hb][db][2], O[hb][db][3]);
      if (g == 0) {
        part_ml[2 * pi] = m[hb];
        part_ml[2 * pi + 1] = l;
      }
    }
  }
}

// ------------------------------------------------------------------ bf16 path
// Same computation for bf16, restructured around two gfx950 instructions:
//  * global_load_lds_dwordx4 gathers key rows from HBM straight into LDS
//    (no staging registers), into a ring of NBUF 64-key tiles, so up to
//    NBUF-1 tiles of gathers are in flight while a tile is computed;
//  * ds_read_b64_tr_b16 reads the V^T fragments of the P*V product
//    transposed out of the same row-major tile, so no transposed copy is built.
// Tiles are 64 rows x 256 B; each row's 16-byte chunk c is stored at position
// c ^ (row & SWM). With SWM = 15, sixteen consecutive rows put any given chunk
// at sixteen different positions, so the K fragment reads (16 rows, one chunk
// each) and the transposed V reads (4 rows x 32 bytes per 16 lanes) spread
// over all LDS banks. A lane of a gather instruction fetches exactly the
// chunk its LDS slot must hold.
constexpr int kSelChunk = 1024;     // selected indices staged in LDS at a time

// One 64-key tile (row-major in LDS, swizzled chunks) for the HPW 16-head
// blocks of one wave: S^T = K Q^T, online softmax against the lazily raised
// running max, O^T += V^T P^T. With `masked`, key_ok(key) says whether tile
// row `key` holds a key; other rows get probability 0 (their LDS rows must
// hold finite values).
template <int HPW, typename KeyOk>
__device__ __forceinline__ void attn_tile16(uint32_t tb, const TileLanes& tl, bool masked, KeyOk key_ok,
                                            const Frag<uint16_t> (&qf)[HPW][kD / 32], float scale2,
                                            float (&m)[HPW], float (&lsum)[HPW], f32x4 (&O)[HPW][kD / 16]) {
  constexpr float kLazy = 8.f;   // headroom of the lazily raised running max (base 2)
  const int g = (threadIdx.x & 63) >> 4;
  // ---- S^T = K Q^T for 4 blocks of 16 keys: 8 independent accumulator
  // chains (key block x head block) over the 4 d-chunks. Logits stay
  // unscaled here; the scale enters the exponent below.
  float s[HPW][4][4];
  {
    f32x4 acc[4][HPW];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int hb = 0; hb < HPW; ++hb) acc[kb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) {
      uint32_t ka = (((uint32_t)(64 * ks)) ^ tl.kx) + (tb + tl.kofs);
      opaque(ka);   // keeps 4096 kb in the reads' offset field
      Frag<uint16_t> a[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) a[kb].v = lds_read_b128(ka + 4096 * kb);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) acc[kb][hb] = mma8(a[kb], qf[hb][ks], acc[kb][hb]);
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int hb = 0; hb < HPW; ++hb) s[hb][kb][rr] = acc[kb][hb][rr];
  }
  if (masked) {   // uniform: only partial or holed tiles are masked
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = 16 * kb + 4 * g + rr;
        if (!key_ok(key)) {
#pragma unroll
          for (int hb = 0; hb < HPW; ++hb) s[hb][kb][rr] = -INFINITY;
        }
      }
  }
  // ---- online softmax (per head = per column), base-2 logits scale2 * s.
  // Lazy rescaling: probabilities are taken against the running reference
  // max m[hb] while no logit of the tile exceeds it by more than kLazy, so
  // P, O and l grow by at most 2^kLazy (exact in float32, and bf16 keeps
  // its relative precision); only a larger logit raises m (the column max
  // over the 4 lane rows, by permlane swaps) and rescales O and l. The
  // result O / l and the log-sum m + log2(l) do not depend on m. One branch
  // (rarely taken) covers every head block, so the exponentials of all head
  // blocks and the P V products that follow form one straight-line block the
  // compiler can interleave.
  float lm2[HPW];
  bool need = false;
#pragma unroll
  for (int hb = 0; hb < HPW; ++hb) {
    float lmax = s[hb][0][0];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) lmax = fmaxf(lmax, s[hb][kb][rr]);
    lm2[hb] = lmax * scale2;
    need |= lm2[hb] > m[hb] + kLazy;
  }
  if (__ballot(need)) {   // wave-uniform, rare: one branch for all head blocks
#pragma unroll
    for (int hb = 0; hb < HPW; ++hb) {
      if (__ballot(lm2[hb] > m[hb] + kLazy)) {
        const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(lm2[hb]), __float_as_uint(lm2[hb]), false, false);
        const float c1 = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
        const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(c1), __float_as_uint(c1), false, false);
        const float cmax = fmaxf(__uint_as_float(y[0]), __uint_as_float(y[1]));
        const float mnew = fmaxf(m[hb], cmax);
        const float alpha = m[hb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[hb] - mnew);
        lsum[hb] *= alpha;
#pragma unroll
        for (int db = 0; db < kD / 16; ++db) O[hb][db] *= alpha;
        m[hb] = mnew;
      }
    }
  }
#pragma unroll
  for (int hb = 0; hb < HPW; ++hb) {
    const float negm = m[hb] == -INFINITY ? 0.f : -m[hb];
    float ps[2] = {0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[hb][kb][rr], scale2, negm));   // exp2(-inf) = 0
        s[hb][kb][rr] = pv;
        ps[rr & 1] += pv;
      }
    lsum[hb] += ps[0] + ps[1];
  }
  // ---- O^T += V^T P^T. K-slot t of lane group g is key 4g+t (t < 4) or
  // 16+4g+(t-4) (t >= 4) of the 32-key group; the transposed reads deliver
  // exactly those keys for value column 16*db + col.
  uint32_t va[kD / 16];
#pragma unroll
  for (int db = 0; db < kD / 16; ++db) {
    va[db] = (((uint32_t)(32 * db)) ^ tl.vx) + (tb + tl.vofs);
    opaque(va[db]);   // keeps 8192 grp + 4096 in the reads' offset field
  }
#pragma unroll
  for (int grp = 0; grp < 2; ++grp) {
    Frag<uint16_t> pf[HPW];
#pragma unroll
    for (int hb = 0; hb < HPW; ++hb) {
      pf[hb].v[0] = (int)cvt_pk_bf16(s[hb][2 * grp][0], s[hb][2 * grp][1]);
      pf[hb].v[1] = (int)cvt_pk_bf16(s[hb][2 * grp][2], s[hb][2 * grp][3]);
      pf[hb].v[2] = (int)cvt_pk_bf16(s[hb][2 * grp + 1][0], s[hb][2 * grp + 1][1]);
      pf[hb].v[3] = (int)cvt_pk_bf16(s[hb][2 * grp + 1][2], s[hb][2 * grp + 1][3]);
    }
#pragma unroll
    for (int db = 0; db < kD / 16; ++db) {
      const s16x4 lo4 = lds_read_tr16(va[db] + 8192 * grp);
      const s16x4 hi4 = lds_read_tr16(va[db] + 8192 * grp + 4096);
      // the 4 + 4 transposed bf16 values already sit in dword order
      const i32x2 l2 = __builtin_bit_cast(i32x2, lo4), h2 = __builtin_bit_cast(i32x2, hi4);
      Frag<uint16_t> vf;
      vf.v = i32x4{l2[0], l2[1], h2[0], h2[1]};
#pragma unroll
      for (int hb = 0; hb < HPW; ++hb) O[hb][db] = mma8(vf, pf[hb], O[hb][db]);
    }
  }
}

template <bool SPARSE, int NW, int HPW, int NBUF, int TS>
__global__ __launch_bounds__(NW * TS * 64, (TS == 1 && NW >= 2) ? 2 : 1) void k_attn16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ x_win, const int32_t* __restrict__ win_start, const float* __restrict__ sink,
    const int32_t* __restrict__ q_pos, int64_t Tq, int64_t N, int64_t T_win, int wring, int H, int k, int window,
    int ratio, float scale, int S, uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  constexpr int NWT = NW * TS;                    // waves: TS streams of NW head waves
  constexpr int NT = NWT * 64;
  constexpr int LPT = (kKT * kD * 2 / 16) / NT;   // 16-byte gathers per thread per tile
  static_assert(NBUF % TS == 0 && NBUF > TS, "ring holds whole tile groups plus prefetch");
  __shared__ __align__(16) uint16_t ring[NBUF][kKT * kD];
  __shared__ int tbadw[NBUF][NWT];   // per wave: its gathers of the slot's tile hit rows without a key
  __shared__ int sidx[SPARSE ? kSelChunk : 1];
  constexpr int QH = NW * HPW * 16;                // query rows (heads) of the block
  constexpr int QPT = QH * 16 / NT;                // 16-byte query gathers per thread
  static_assert(QPT * NT == QH * 16, "query rows split evenly over the threads");
  // two tile streams (few rows, short key ranges): the query goes through LDS
  __shared__ __align__(16) uint16_t qs[TS > 1 ? QH * kD : 8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // 0 .. NWT-1: gathers
  const int hw = wv % NW, ts = wv / NW;                      // head wave, tile stream
  const int g = lane >> 4, col = lane & 15;
  constexpr int SWM = 15;                         // chunk swizzle mask of the tiles
  const TileLanes tl(lane, SWM);
  // rows < 2^31: 32-bit row arithmetic, so that both scalar loads below are
  // issued together (a 64-bit division would put a branch between them)
  const int32_t r32 = blockIdx.x, b32 = r32 / (int32_t)Tq;
  const int64_t r = r32, b = b32;
  const int hg = blockIdx.y / S, sp = blockIdx.y % S;
  // Selected indices [c0, c0 + cnt) of the row copied to LDS, one dword per
  // lane, all copies in flight together (slots past the selected entries
  // belong to window keys and are never read).
  auto stage_sel = [&](int64_t c0, int cnt) {
    const int32_t* isrc = idx + r * k + c0;
    for (int j = 0; j * NT < cnt; ++j) {
      const int i = j * NT + wv * 64 + lane;
      if (i < cnt) gather_lds4_s(isrc, 4u * (uint32_t)i, (uint32_t)(uintptr_t)(sidx + j * NT + wv * 64));
    }
  };
  // With one split the first section starts at the row's first selected
  // entry whatever the query position: its indices need no loaded value.
  if (SPARSE && S == 1) stage_sel(0, k < kSelChunk ? k : kSelChunk);
  if constexpr (TS > 1) {
    // the query gathers go first: their addresses need no loaded value
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
      const int qrow = (j * NWT + wv) * 4 + (lane >> 4);
      gather_lds16(q + (r * H + hg * QH + qrow) * kD + (((lane & 15) ^ (qrow & SWM)) << 3),
                   (uint32_t)(uintptr_t)(qs + (j * NWT + wv) * 4 * kD));
    }
  }
  const int32_t w0_32 = win_start[b32];
  const int32_t p32 = q_pos[r32];
  const int64_t p = p32, w0 = w0_32;
  const int64_t n_sel = SPARSE ? (int64_t)k : visible(p32, ratio, N);
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
  // row of window position lo: lo - w0, or lo mod T_win for a ring (a window
  // of at most T_win rows wraps at most once)
  const int64_t wrow0 = wring ? lo % (T_win > 0 ? T_win : 1) : lo - w0;

  const int h0 = hg * QH + hw * 16 * HPW;
  // With two tile streams (short key ranges per block) the query rows go to
  // LDS by the same asynchronous gathers as the keys, issued first so that the
  // first wait on key tiles covers them, and the waves read their fragments
  // from there: no vector load that the compiler tracks (and would wait for,
  // draining the key pipeline) precedes the first tile. With one stream the
  // fragments are loaded directly and waited for before the first gather.
  Frag<uint16_t> qf[HPW][kD / 32];
  if constexpr (TS == 1) {
#pragma unroll
    for (int hb = 0; hb < HPW; ++hb) {
      const uint16_t* qrow = q + (r * H + h0 + 16 * hb + col) * kD;
#pragma unroll
      for (int ks = 0; ks < kD / 32; ++ks) qf[hb][ks].load(qrow + 32 * ks + 8 * g);
    }
    if (!SPARSE) wait_vm<0>();   // the sparse path waits after its index staging
  }
  auto load_q = [&]() {
    if constexpr (TS > 1) {
#pragma unroll
      for (int hb = 0; hb < HPW; ++hb)
#pragma unroll
        for (int ks = 0; ks < kD / 32; ++ks)
          qf[hb][ks].v = lds_read_b128((uint32_t)(uintptr_t)qs + (hw * HPW + hb) * 4096 + tl.kofs + ((64u * ks) ^ tl.kx));
    }
  };
  // Logits are kept in base 2 (log2(e) folded into the scale) so each
  // probability is one v_exp_f32.
  constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
  const float scale2 = scale * kLog2e;
  float m[HPW], lsum[HPW];
  f32x4 O[HPW][kD / 16];
#pragma unroll
  for (int hb = 0; hb < HPW; ++hb) {
    m[hb] = -INFINITY;
    lsum[hb] = 0.f;
#pragma unroll
    for (int db = 0; db < kD / 16; ++db) O[hb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint16_t* dummy = q + r * H * kD;   // a finite row for slots without a key
  // entry byte offsets fit 32 bits (and entry 0 exists)
  const bool offs32 = N >= 1 && N <= ((int64_t)1 << 24);
  const uint16_t* kvb = kv + b * N * kD;
  const uint16_t* xwb = x_win + b * T_win * kD;

  // Keys are processed in sections of up to kSelChunk (the selected indices
  // of a section are staged in LDS first), each as a pipeline of 64-key tiles.
  for (int64_t c0 = kbeg; c0 < kend; c0 += kSelChunk) {
    const int clen = (int)((kend - c0) < kSelChunk ? (kend - c0) : kSelChunk);
    if (SPARSE) {
      // The section's selected indices go straight to LDS (with one split
      // the first section's were issued at entry).
      if (!(S == 1 && c0 == 0)) stage_sel(c0, (int)(n_sel - c0 < (int64_t)clen ? n_sel - c0 : (int64_t)clen));
      wait_vm<0>();   // every thread: the query and index loads are done before any gather
      __syncthreads();
      if (c0 == kbeg) load_q();
    }
    const int ntiles = (clen + kKT - 1) / kKT;
    // Keys [0, sel_end) of the section are entries (selected or dense), the
    // rest window rows; window row of key kk >= sel_end: wbase + kk, less
    // T_win once past the end of a ring.
    const int64_t se = n_sel - c0;
    const int sel_end = se <= 0 ? 0 : (se < (int64_t)clen ? (int)se : clen);
    const int64_t wbase = wrow0 - se;
    // Gather instruction j of this lane: tile row grow(j) (4 rows per wave
    // instruction), 16-byte chunk gcol(j) of it (swizzled position lane & 15):
    // grow(j) mod 16 = 4 ((j NWT + wv) mod 4) + lane / 16, and (j NWT + wv)
    // mod 4 = (j NWT mod 4) ^ (wv mod 4) for the wave counts used, so the
    // chunk is one per-lane value xor a constant of j (no per-j registers).
    static_assert(NWT == 1 || NWT == 2 || NWT % 4 == 0, "gather row pattern");
    const int gc0 = ((lane & 15) ^ (((wv & 3) << 2) | (lane >> 4))) << 3;
    auto grow = [&](int j) { return (j * NWT + wv) * 4 + (lane >> 4); };
    auto gcol = [&](int j) { return gc0 ^ (((j * NWT) & 3) << 5); };
    // whether key kk of the section holds a key: inside the section and, for a
    // selected entry, an index in [0, N)
    const uint32_t n32 = N < ((int64_t)1 << 31) ? (uint32_t)N : 0x80000000u;
    auto key_ok = [&](int kk) {
      if constexpr (SPARSE) return kk < clen && (kk >= sel_end || (uint32_t)sidx[kk] < n32);
      else return kk < clen;
    };
    auto issue = [&](int t) {
      const int slot = t % NBUF;
      uint16_t* base = ring[slot];
      const int kk0 = t * kKT;
      const int nt = (clen - kk0) < kKT ? (clen - kk0) : kKT;   // keys of the tile
      bool bad = false;
      int64_t wt = wbase + kk0;   // window row of the tile's first key (window tiles)
      if (wt >= T_win) wt -= T_win;
      const bool win_run = kk0 >= sel_end && wt + nt <= T_win;
      if (win_run || (!SPARSE && kk0 + nt <= sel_end)) {
        // the tile's keys are consecutive rows: window rows (not wrapping
        // around a ring), or dense entries; the rows of a partial tile past
        // its last key repeat that key (masked)
        const uint16_t* tb = win_run ? xwb + wt * kD : kvb + (c0 + kk0) * kD;
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
          const int row = grow(j) < nt ? grow(j) : nt - 1;
          gather_lds16_s(tb, (uint32_t)row * (uint32_t)(kD * 2) + (uint32_t)gcol(j) * 2u,
                         (uint32_t)(uintptr_t)(base + (j * NWT + wv) * 4 * kD));
        }
      } else if (SPARSE && offs32 && kk0 + kKT <= sel_end) {
        // 64 selected entries: byte offsets from the batch's first entry (an
        // entry outside [0, N) reads entry 0 and is marked). All index reads
        // go first: a gather statement orders memory accesses around it, so
        // a read placed between gathers would be waited for one at a time.
        int32_t ent[LPT];
#pragma unroll
        for (int j = 0; j < LPT; ++j) ent[j] = sidx[kk0 + grow(j)];
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
          const int32_t e = ent[j];
          const bool ok = (uint32_t)e < n32;
          bad |= !ok;
          gather_lds16_s(kvb, (ok ? (uint32_t)e * (uint32_t)(kD * 2) : 0u) + (uint32_t)gcol(j) * 2u,
                         (uint32_t)(uintptr_t)(base + (j * NWT + wv) * 4 * kD));
        }
      } else {
        // entries and window rows mixed, a window run that wraps, or entries
        // past 2^24: one address per gather; rows past the section's end
        // repeat its last key and an entry outside [0, N) reads a finite row
        // (both masked)
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
          const int kk = (kk0 + grow(j)) < clen ? kk0 + grow(j) : clen - 1;
          const uint16_t* src;
          if (kk < sel_end) {
            const int64_t e = SPARSE ? (int64_t)sidx[kk] : c0 + kk;
            const bool ok = e >= 0 && e < N;
            bad |= !ok;
            src = ok ? kvb + e * kD : dummy;
          } else {
            int64_t wr = wbase + kk;
            if (wr >= T_win) wr -= T_win;
            src = xwb + wr * kD;
          }
          gather_lds16(src + gcol(j), (uint32_t)(uintptr_t)(base + (j * NWT + wv) * 4 * kD));
        }
      }
      const bool wbad = __ballot(bad) != 0ull;
      if (lane == 0) tbadw[slot][wv] = wbad;
    };
    // Tiles are taken TS at a time (stream ts computes tile t0 + ts); the
    // gathers of the next NBUF - TS tiles stay in flight meanwhile.
#pragma unroll
    for (int t = 0; t < NBUF - TS; ++t)
      if (t < ntiles) issue(t);
    if (!SPARSE && TS > 1 && c0 == kbeg) {
      // the query gathers are older than the key gathers just issued
      if (ntiles >= NBUF - TS) wait_vm<(NBUF - TS) * LPT>();
      else wait_vm<0>();
      __syncthreads();
      load_q();
    }

    for (int t0 = 0; t0 < ntiles; t0 += TS) {
#pragma unroll
      for (int j = 0; j < TS; ++j)
        if (t0 + NBUF - TS + j < ntiles) issue(t0 + NBUF - TS + j);
      if (t0 + NBUF - 1 < ntiles) wait_vm<(NBUF - TS) * LPT>();
      else wait_vm<0>();
      __syncthreads();
      const int t = t0 + ts;
      if (t < ntiles) {   // uniform per wave
      const int slot = t % NBUF;
      const uint32_t tb = (uint32_t)(uintptr_t)ring[slot];
      const int nt = (clen - t * kKT) < kKT ? (clen - t * kKT) : kKT;

      bool holed = false;
#pragma unroll
      for (int w = 0; w < NWT; ++w) holed |= tbadw[slot][w] != 0;
      // slots without a key hold a finite row (the query's) and get probability 0
      attn_tile16<HPW>(tb, tl, nt < kKT || holed, [&](int key) { return key_ok(t * kKT + key); }, qf, scale2,
                       m, lsum, O);
      }   // t < ntiles
      __syncthreads();   // the slots are refilled by later issue() calls
    }
  }
  wait_vm<0>();   // a block without keys still has its query gathers in flight

  if constexpr (TS > 1) {
    // Stream 1 hands (O, m, lsum) to stream 0 through the (now idle) ring, in
    // lane order; stream 0 merges: every value is rescaled to the larger max.
    static_assert(TS == 2, "two tile streams");
    static_assert(NW * HPW * (kD / 16) * 64 * 4 * 4 + NW * HPW * 64 * 2 * 4 <= NBUF * kKT * kD * 2, "exchange fits");
    float* xo = reinterpret_cast<float*>(&ring[0][0]);
    float* xml = xo + NW * HPW * (kD / 16) * 64 * 4;
    if (ts == 1) {
#pragma unroll
      for (int hb = 0; hb < HPW; ++hb) {
#pragma unroll
        for (int db = 0; db < kD / 16; ++db)
          *reinterpret_cast<f32x4*>(xo + (((hw * HPW + hb) * (kD / 16) + db) * 64 + lane) * 4) = O[hb][db];
        xml[((hw * HPW + hb) * 64 + lane) * 2] = m[hb];
        xml[((hw * HPW + hb) * 64 + lane) * 2 + 1] = lsum[hb];
      }
    }
    __syncthreads();
    if (ts == 1) return;
#pragma unroll
    for (int hb = 0; hb < HPW; ++hb) {
      const float m1 = xml[((hw * HPW + hb) * 64 + lane) * 2], l1 = xml[((hw * HPW + hb) * 64 + lane) * 2 + 1];
      const float mm = fmaxf(m[hb], m1);
      const float a0 = m[hb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[hb] - mm);
      const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
      lsum[hb] = lsum[hb] * a0 + l1 * a1;
      m[hb] = mm;
#pragma unroll
      for (int db = 0; db < kD / 16; ++db) {
        const f32x4 o1 = *reinterpret_cast<const f32x4*>(xo + (((hw * HPW + hb) * (kD / 16) + db) * 64 + lane) * 4);
        O[hb][db] = O[hb][db] * a0 + o1 * a1;
      }
    }
  }

  // O's factor at the output (the sink's rescale of O is folded into it)
  float osc[HPW];
#pragma unroll
  for (int hb = 0; hb < HPW; ++hb) osc[hb] = 1.f;
  if (sink != nullptr && sp == 0) {
    // The sink is one more logit (value 0) of split 0: it joins the
    // denominator, with the running max raised to it when larger.
#pragma unroll
    for (int hb = 0; hb < HPW; ++hb) {
      const float ms = sink[h0 + 16 * hb + col] * kLog2e;
      const float mm = fmaxf(m[hb], ms);
      const float a0 = m[hb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[hb] - mm);
      lsum[hb] = lsum[hb] * a0 + (g == 0 ? __builtin_amdgcn_exp2f(ms - mm) : 0.f);
      m[hb] = mm;
      osc[hb] = a0;
    }
  }

#pragma unroll
  for (int hb = 0; hb < HPW; ++hb) {
    float l = lsum[hb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int head = h0 + 16 * hb + col;
    // The output (one split) or this split's partial result: the softmax
    // average O / l in bf16, rounded to nearest even (v_cvt_pk_bf16_f32; a
    // partial is combined convexly by the merge, so its rounding stays within
    // that of the bf16 output). The head block's 16 rows go through a
    // wave-private piece of the idle ring (rows padded to 272 bytes against
    // bank conflicts; with two tile streams, inside this wave's own block of
    // the exchange area), so that each head's 256-byte row leaves in one
    // store instruction of 16-byte pieces (4 stores per lane instead of 8 of
    // 8 bytes, whole lines).
    const float inv = l > 0.f ? osc[hb] / l : 0.f;
    constexpr int kXs = 136;   // staged row stride (elements)
    static_assert((TS > 1 ? HPW * 4096 : 16 * kXs) * NW <= NBUF * kKT * kD, "staging fits the ring");
    uint16_t* xs = &ring[0][0] + hw * (TS > 1 ? HPW * 4096 : 16 * kXs);
#pragma unroll
    for (int db = 0; db < kD / 16; ++db)
      *reinterpret_cast<uint2*>(xs + col * kXs + 16 * db + 4 * g) =
          make_uint2(cvt_pk_bf16(O[hb][db][0] * inv, O[hb][db][1] * inv), cvt_pk_bf16(O[hb][db][2] * inv, O[hb][db][3] * inv));
    uint16_t* dst = S == 1 ? out + (r * H + h0 + 16 * hb) * kD
                           : reinterpret_cast<uint16_t*>(part_o) + ((r * H + h0 + 16 * hb) * S + sp) * kD;
    const int64_t hstride = S == 1 ? kD : (int64_t)S * kD;   // elements between the block's head rows
#pragma unroll
    for (int j = 0; j < 4; ++j) {   // piece lane & 15 of head row 4 j + lane / 16
      const int hh = 4 * j + (lane >> 4), c = lane & 15;
      const uint4 v = *reinterpret_cast<const uint4*>(xs + hh * kXs + 8 * c);
      *reinterpret_cast<uint4*>(dst + hh * hstride + 8 * c) = v;
    }
    if (S == 1) {
      if (lse && g == 0) lse[r * H + head] = l > 0.f ? (m[hb] + __log2f(l)) * kLn2 : -INFINITY;
    } else if (g == 0) {
      const int64_t pi = (r * H + head) * S + sp;
      part_ml[2 * pi] = m[hb] * kLn2;   // the merge works in natural-log units
      part_ml[2 * pi + 1] = l;
    }
  }
}

// Merge of S partial results per (row, head), in split order. 32 lanes x 4
// channels per (row, head) pair, blockDim / 32 pairs per block. The splits are taken in
// chunks of CH whose loads are all issued before any is used (one memory
// round trip per chunk); a chunk is folded into the running (max, sum, O)
// in split order. Partials are unnormalised float sums (PT = float) or
// bf16 split averages O / l (PT = uint16_t); (m, l) are float, m in
// natural-log units.
template <typename T, typename PT>
__global__ __launch_bounds__(256) void k_attn_merge(const PT* __restrict__ part_o, const float* __restrict__ part_ml,
                                                    int64_t RH, int S, T* __restrict__ out, float* __restrict__ lse) {
  constexpr int CH = sizeof(PT) == 2 ? 32 : 16;
  const int64_t rh = (int64_t)blockIdx.x * (blockDim.x >> 5) + (threadIdx.x >> 5);
  const int d0 = (threadIdx.x & 31) * 4;
  if (rh >= RH) return;
  const float2* ml = reinterpret_cast<const float2*>(part_ml) + rh * S;
  float M = -INFINITY, l = 0.f;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < S; c0 += CH) {
    const int n = S - c0 < CH ? S - c0 : CH;
    float2 mv[CH];
    float v[CH][4];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      mv[j] = j < n ? ml[c0 + j] : make_float2(-INFINITY, 0.f);
      if constexpr (sizeof(PT) == 2) {
        const uint2 u = j < n ? *reinterpret_cast<const uint2*>(part_o + (rh * S + c0 + j) * kD + d0) : make_uint2(0, 0);
        v[j][0] = __uint_as_float(u.x << 16); v[j][1] = __uint_as_float(u.x & 0xffff0000u);
        v[j][2] = __uint_as_float(u.y << 16); v[j][3] = __uint_as_float(u.y & 0xffff0000u);
      } else {
        const float4 u = j < n ? *reinterpret_cast<const float4*>(part_o + (rh * S + c0 + j) * kD + d0)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
        v[j][0] = u.x; v[j][1] = u.y; v[j][2] = u.z; v[j][3] = u.w;
      }
    }
    float cm = -INFINITY;
#pragma unroll
    for (int j = 0; j < CH; ++j) cm = fmaxf(cm, mv[j].x);
    if (cm == -INFINITY) continue;   // uniform per pair
    const float mn = fmaxf(M, cm);
    const float a = M == -INFINITY ? 0.f : __expf(M - mn);
    l *= a;
    o[0] *= a; o[1] *= a; o[2] *= a; o[3] *= a;
    M = mn;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const float e = mv[j].x == -INFINITY ? 0.f : __expf(mv[j].x - M);
      float f;
      if constexpr (sizeof(PT) == 2) {
        f = e * mv[j].y;   // weight of the split average
        l += f;
      } else {
        f = e;
        l = fmaf(mv[j].y, e, l);
      }
      o[0] = fmaf(v[j][0], f, o[0]); o[1] = fmaf(v[j][1], f, o[1]);
      o[2] = fmaf(v[j][2], f, o[2]); o[3] = fmaf(v[j][3], f, o[3]);
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float r[4] = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
  Elem<T>::store4(out + rh * kD + d0, r);
  if (lse && d0 == 0) lse[rh] = l > 0.f ? M + __logf(l) : -INFINITY;
}

// ------------------------------------------------------------------ host side

// Waves per block and 16-head blocks per wave: 2 head blocks per wave when
// possible (each LDS fragment then feeds two MFMAs), up to 4 waves.
struct AttnShape { int nw, hpw; };
static AttnShape pick_shape(int H) {
  const int hb = H / 16;
  const int hpw = (hb % 2 == 0) ? 2 : 1;
  const int waves = hb / hpw;
  const int nw = (waves % 4 == 0) ? 4 : (waves % 2 == 0 ? 2 : 1);
  return {nw, hpw};
}

// Key splits per (row, head group): a fixed function of the shapes (never of
// timing), so the workspace query and the launch agree and the merge order is
// fixed. About one block per compute unit, >= kMinSplitKeys keys per split.
constexpr int64_t kMinSplitKeys = 128;
static int split_count(int64_t rows, int H, AttnShape sh, int64_t nk_max) {
  const int64_t base = rows * (H / (16 * sh.nw * sh.hpw));
  if (base >= 256) return 1;
  const int64_t fill = cdiv(256, base);
  const int64_t by_keys = nk_max / kMinSplitKeys > 1 ? nk_max / kMinSplitKeys : 1;
  int64_t s = fill < by_keys ? fill : by_keys;
  if (s > 128) s = 128;
  return (int)(s < 1 ? 1 : s);
}

// Short splits (at most kShortSplitKeys keys, five 64-key tiles: a decode
// grid split across the keys): one head block per wave instead of two when
// that doubles the blocks per row, which halves the splits. A block's fixed
// costs (query load, output staging, partial writes) then weigh on half as
// many heads and the merge reads half the partials; long splits keep two
// head blocks per wave, whose shared key fragments save more than the extra
// blocks gain (measured on 128 heads: sparse decode over 1,152 keys per row
// is faster at 8 to 64 rows, dense decode over 8,320 keys only at 8).
constexpr int64_t kShortSplitKeys = 320;
struct AttnPlan { int S; AttnShape sh; };
static AttnPlan plan_attention(int64_t rows, int H, int64_t nk_max) {
  AttnShape sh = pick_shape(H);
  int S = split_count(rows, H, sh, nk_max);
  if (S > 1 && sh.hpw == 2 && sh.nw == 4 && nk_max <= kShortSplitKeys * S) {
    sh.hpw = 1;
    S = split_count(rows, H, sh, nk_max);
  }
  return {S, sh};
}

// Batch-invariant planning (a per-call option): the split count and the
// tile-stream choice follow one sequence's rows (Tq) instead of the whole
// batch (B * Tq), so a sequence's result does not depend on what else is in
// the batch.
static int64_t plan_rows(int64_t B, int64_t Tq, bool batch_inv) { return batch_inv ? Tq : B * Tq; }

int attn_splits(int64_t rows, int H, int64_t nk_max) { return plan_attention(rows, H, nk_max).S; }

size_t attn_ws_bytes(int64_t B, int64_t Tq, int H, int64_t nk_max, bool batch_inv) {
  const int S = attn_splits(plan_rows(B, Tq, batch_inv), H, nk_max);
  if (S == 1) return 0;
  return (size_t)(B * Tq) * H * S * (kD + 2) * 4;
}

// (row, head) pairs per merge block: 2 to 8, about 512 blocks (the few pairs
// of a decode step spread over more compute units than 8 per block allow)
static int merge_pairs(int64_t RH) {
  int p = 2;
  while (p < 8 && RH / (2 * p) >= 512) p *= 2;
  return p;
}

constexpr int kRing = 2;   // ring slots per block (bf16 path, one tile stream): a small ring leaves LDS
                           // for more resident blocks, which hides more latency than deeper prefetch
constexpr int kRing2 = 6;  // ring slots with two tile streams (2 computed + 4 in flight)

template <typename T, bool SPARSE, int NW, int HPW>
static void launch_attn_t(dim3 grid, hipStream_t st, const void* q, const void* kv, const int32_t* idx,
                          const void* x_win, const int32_t* win_start, const float* sink, const int32_t* q_pos,
                          int64_t Tq, int64_t N, int64_t T_win, int wring, int H, int k, int window, int ratio,
                          float scale, int S, bool two_streams, void* out, float* lse, float* po, float* pml) {
  if constexpr (sizeof(T) == 2) {
    // Few rows (decode): two tile streams per block, two waves per SIMD.
    if (two_streams)
      k_attn16<SPARSE, NW, HPW, kRing2, 2><<<grid, NW * 2 * 64, 0, st>>>(
          (const uint16_t*)q, (const uint16_t*)kv, idx, (const uint16_t*)x_win, win_start, sink, q_pos, Tq, N, T_win,
          wring, H, k, window, ratio, scale, S, (uint16_t*)out, lse, po, pml);
    else
      k_attn16<SPARSE, NW, HPW, kRing, 1><<<grid, NW * 64, 0, st>>>(
          (const uint16_t*)q, (const uint16_t*)kv, idx, (const uint16_t*)x_win, win_start, sink, q_pos, Tq, N, T_win,
          wring, H, k, window, ratio, scale, S, (uint16_t*)out, lse, po, pml);
  }
  else
    k_attn<T, SPARSE, NW, HPW><<<grid, NW * 64, 0, st>>>((const T*)q, (const T*)kv, idx, (const T*)x_win, win_start,
                                                         sink, q_pos, Tq, N, T_win, wring, H, k, window, ratio, scale,
                                                         S, (T*)out, lse, po, pml);
}

template <typename T, bool SPARSE>
static void launch_attn_sh(AttnShape sh, dim3 grid, hipStream_t st, const void* q, const void* kv, const int32_t* idx,
                           const void* x_win, const int32_t* win_start, const float* sink, const int32_t* q_pos,
                           int64_t Tq, int64_t N, int64_t T_win, int wring, int H, int k, int window, int ratio,
                           float scale, int S, bool two_streams, void* out, float* lse, float* po, float* pml) {
#define CSA_ATTN_CASE(NW_, HPW_)                                                                               \
  if (sh.nw == NW_ && sh.hpw == HPW_) {                                                                        \
    launch_attn_t<T, SPARSE, NW_, HPW_>(grid, st, q, kv, idx, x_win, win_start, sink, q_pos, Tq, N, T_win,    \
                                        wring, H, k, window, ratio, scale, S, two_streams, out, lse, po, pml);  \
    return;                                                                                                    \
  }
  CSA_ATTN_CASE(4, 2)
  CSA_ATTN_CASE(2, 2)
  CSA_ATTN_CASE(1, 2)
  CSA_ATTN_CASE(4, 1)
  CSA_ATTN_CASE(2, 1)
  CSA_ATTN_CASE(1, 1)
#undef CSA_ATTN_CASE
}

// One row of 128 elements per sequence into ring row pos mod R (16 bytes per thread).
template <typename T>
__global__ __launch_bounds__(256) void k_window_append(const T* __restrict__ x_new, int64_t B,
                                                       const int32_t* __restrict__ pos, T* __restrict__ ring,
                                                       int64_t R) {
  constexpr int C = 16 / sizeof(T);                 // elements per 16-byte chunk
  constexpr int CPR = kD / C;                       // chunks per row
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= B * CPR) return;
  const int64_t b = i / CPR, c = i % CPR;
  if (pos[b] < 0) return;   // a negative position skips the sequence
  const int64_t row = (int64_t)((uint32_t)pos[b] % (uint64_t)R);
  *reinterpret_cast<i32x4*>(ring + (b * R + row) * kD + c * C) =
      *reinterpret_cast<const i32x4*>(x_new + b * kD + c * C);
}

hipError_t launch_window_append(const void* x_new, csa_dtype t, int64_t B, const int32_t* pos, void* ring,
                                int64_t R, hipStream_t s) {
  if (t == CSA_BF16) {
    const int64_t n = B * (kD / 8);
    k_window_append<uint16_t><<<(unsigned)cdiv(n, 256), 256, 0, s>>>(static_cast<const uint16_t*>(x_new), B, pos,
                                                                      static_cast<uint16_t*>(ring), R);
  } else {
    const int64_t n = B * (kD / 4);
    k_window_append<float><<<(unsigned)cdiv(n, 256), 256, 0, s>>>(static_cast<const float*>(x_new), B, pos,
                                                                   static_cast<float*>(ring), R);
  }
  return hipGetLastError();
}

hipError_t launch_attention(bool sparse, csa_dtype t, const void* q, const void* kv, const int32_t* idx,
                            const void* x_win, const int32_t* win_start, const float* sink, const int32_t* q_pos,
                            int64_t B, int64_t Tq, int64_t N, int64_t T_win, int wring, int H, int k, int window,
                            int ratio, float scale, void* out, float* lse, void* ws, int64_t nk_max, bool batch_inv,
                            hipStream_t st) {
  const int64_t rows = B * Tq;
  if (rows == 0) return hipSuccess;
  const int64_t prow = plan_rows(B, Tq, batch_inv);
  const AttnPlan pl = plan_attention(prow, H, nk_max);
  const AttnShape sh = pl.sh;
  const int S = pl.S;
  // two tile streams when the planned grid is small (few rows: decode)
  const bool two_streams = prow * (H / (16 * sh.nw * sh.hpw)) * S <= 1024;
  float* po = reinterpret_cast<float*>(ws);
  float* pml = po ? po + (size_t)rows * H * S * kD : nullptr;
  const dim3 grid((unsigned)rows, (unsigned)((H / (16 * sh.nw * sh.hpw)) * S));
  const int kid = sparse ? CSA_KID_SPARSE_ATTN : CSA_KID_DENSE_ATTN;
  timer_before(kid, st);
  if (t == CSA_BF16) {
    if (sparse) launch_attn_sh<uint16_t, true>(sh, grid, st, q, kv, idx, x_win, win_start, sink, q_pos, Tq, N, T_win, wring, H, k, window, ratio, scale, S, two_streams, out, lse, po, pml);
    else launch_attn_sh<uint16_t, false>(sh, grid, st, q, kv, idx, x_win, win_start, sink, q_pos, Tq, N, T_win, wring, H, k, window, ratio, scale, S, two_streams, out, lse, po, pml);
  } else {
    if (sparse) launch_attn_sh<float, true>(sh, grid, st, q, kv, idx, x_win, win_start, sink, q_pos, Tq, N, T_win, wring, H, k, window, ratio, scale, S, two_streams, out, lse, po, pml);
    else launch_attn_sh<float, false>(sh, grid, st, q, kv, idx, x_win, win_start, sink, q_pos, Tq, N, T_win, wring, H, k, window, ratio, scale, S, two_streams, out, lse, po, pml);
  }
  hipError_t e = hipGetLastError();
  timer_after(kid, st);
  if (e != hipSuccess || S == 1) return e;
  const int64_t RH = rows * H;
  timer_before(CSA_KID_ATTN_MERGE, st);
  if (t == CSA_BF16)   // the bf16 kernels leave bf16 split averages
    k_attn_merge<uint16_t, uint16_t><<<dim3((unsigned)cdiv(RH, merge_pairs(RH))), 32 * merge_pairs(RH), 0, st>>>(
        reinterpret_cast<const uint16_t*>(po), pml, RH, S, (uint16_t*)out, lse);
  else
    k_attn_merge<float, float><<<dim3((unsigned)cdiv(RH, merge_pairs(RH))), 32 * merge_pairs(RH), 0, st>>>(po, pml, RH, S, (float*)out, lse);
  e = hipGetLastError();
  timer_after(CSA_KID_ATTN_MERGE, st);
  return e;
}

}  // namespace csa
