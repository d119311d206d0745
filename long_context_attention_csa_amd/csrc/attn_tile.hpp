// MFMA fragments and LDS tile addressing shared by the attention forward and
// backward kernels (bf16 and float32 operands, 16x16 MFMA tiles, 64-key tiles
// of 128-element rows in LDS with XOR-swizzled 16-byte chunks).
#pragma once
#include "common.hpp"

namespace csa {

constexpr int kKT = 64;            // keys per tile
constexpr int kD = 128;            // head dim

// 8 consecutive K-elements of one lane's MFMA operand.
template <typename T> struct Frag;
template <> struct Frag<uint16_t> {
  i32x4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const i32x4*>(p); }
  __device__ __forceinline__ void store(uint16_t* p) const { *reinterpret_cast<i32x4*>(p) = v; }
  __device__ __forceinline__ void zero() { v = i32x4{0, 0, 0, 0}; }
  __device__ __forceinline__ uint32_t elem(int j) const {
    const uint32_t w = (uint32_t)v[j >> 1];
    return (j & 1) ? (w >> 16) : (w & 0xffffu);
  }
  // keys {0..3} from p, {4..7} from q
  __device__ __forceinline__ void load_split(const uint16_t* p, const uint16_t* q) {
    const uint2 a = *reinterpret_cast<const uint2*>(p);
    const uint2 b = *reinterpret_cast<const uint2*>(q);
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
  __device__ __forceinline__ void load_split(const float* p, const float* q) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(q);
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

// Per-lane byte offsets of a wave's reads of one tile (the same for every
// tile). K fragment (key block kb, d-step ks) of lane (g, col): row 16 kb + col,
// chunk 4 ks + g, at byte kofs + ((64 ks) ^ kx) + 4096 kb. Transposed V read
// (key half grp, 16-key half hi, d block db): row 32 grp + 16 hi + trow with
// trow = 4 g + col / 4, 8 bytes of chunk 2 db + (col & 3) / 2, at byte
// vofs + ((32 db) ^ vx) + 8192 grp + 4096 hi.
struct TileLanes {
  uint32_t kofs, kx, vofs, vx;
  __device__ __forceinline__ TileLanes(int lane, int swm) {
    const int g = lane >> 4, col = lane & 15;
    kofs = col * 256 + 16 * ((g ^ col) & 3);
    kx = 64 * ((col & swm) >> 2);
    const int trow = 4 * g + (col >> 2), tc = col & 3;
    vofs = trow * 256 + 16 * (((tc >> 1) ^ trow) & 1) + 8 * (tc & 1);
    vx = 32 * ((trow & swm) >> 1);
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ s16x4 lds_read_tr16(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t)a);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

}  // namespace csa
