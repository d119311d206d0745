// Internal helpers shared by the HIP kernels of libcsa_hip (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa_hip.h"
#include "../../include/csa_hip_timer.h"

namespace csa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// float32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Load 8 consecutive elements as float (from float32 or bf16 storage).
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static void load8(const float* p, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ static void store8(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  __device__ __forceinline__ static void store4(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static void load8(const uint16_t* p, float* v) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void store8(uint16_t* p, const float* v) {
    uint4 a;
    a.x = pack_bf16x2(v[0], v[1]); a.y = pack_bf16x2(v[2], v[3]);
    a.z = pack_bf16x2(v[4], v[5]); a.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = a;
  }
  __device__ __forceinline__ static void store4(uint16_t* p, const float* v) {
    uint2 a;
    a.x = pack_bf16x2(v[0], v[1]); a.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(p) = a;
  }
};

// ------------------------------------------------------------------ fp8 / fp4 codes
// OCP e4m3: bias 7, 3 mantissa bits, max 448 (0x7E), 0x7F = NaN.
// Round to nearest even on the float32 value, saturating at 448; the sign bit
// follows the input's sign.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (!(a < 448.0f)) {
    code = (a != a) ? 0x7fu : 0x7eu;
  } else if (a < 0.015625f) {            // below 2^-6: multiples of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);   // exact scaling, RNE
  } else {
    const uint32_t au = __float_as_uint(a);
    const int e = (int)(au >> 23) - 127;
    const uint32_t mf = au & 0x7fffffu;
    uint32_t r = mf >> 20;
    const uint32_t rem = mf & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
    code = (uint32_t)((e + 7) << 3) + r;  // a mantissa carry moves into the exponent
    if (code > 0x7eu) code = 0x7eu;
  }
  return code | sign;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = (e == 0) ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -v : v;
}

// e2m1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}: nearest, ties to the even code, saturating.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  const float a = fabsf(v);
  uint32_t mag;
  if (a <= 0.25f) mag = 0;
  else if (a < 0.75f) mag = 1;
  else if (a <= 1.25f) mag = 2;
  else if (a < 1.75f) mag = 3;
  else if (a <= 2.5f) mag = 4;
  else if (a < 3.5f) mag = 5;
  else if (a <= 5.0f) mag = 6;
  else mag = 7;
  return mag | ((__float_as_uint(v) >> 28) & 8u);
}

// floor(log2(a)) for a finite a > 0 (normal or subnormal).
__device__ __forceinline__ int floor_log2f(float a) {
  const uint32_t u = __float_as_uint(a);
  const int e = (int)((u >> 23) & 0xffu);
  if (e != 0) return e - 127;
  return (31 - __clz((int)(u & 0x7fffffu))) - 149;
}

// Shared exponent of an MX block (E8M0 value minus 127) from the block amax.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int E = floor_log2f(amax) - 2;
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

// 2^k for k in [-126, 127] as an exact float.
__device__ __forceinline__ float pow2i(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

// ------------------------------------------------------------------ selection keys
// Order-preserving map float32 -> uint32 (larger float <-> larger key), with
// -0 mapped like +0.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------------ LDS staging
typedef __attribute__((address_space(3))) const i32x4 lds_i32x4;
// Hides a value from the optimiser, so that constant offsets added to it are
// not reassociated into separately hoisted registers.
__device__ __forceinline__ void opaque(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ i32x4 lds_read_b128(uint32_t a) { return *(lds_i32x4*)(size_t)a; }

// One global_load_lds_dwordx4: each lane's 16 bytes at src go to LDS address
// lds_base + 16 * lane. Written as asm so that the compiler does not treat it
// as an LDS store: it would otherwise drain every outstanding load before
// each later LDS access or barrier (it cannot tell the ring slots apart),
// which serialises the staging pipeline. Completion is tracked explicitly
// with wait_vm() followed by a barrier before a slot is read. The LDS base
// goes through M0, which the compiler reserves: each statement saves M0 in a
// scratch SGPR and restores it after the issue (the instruction reads M0 when
// it is issued), so no value the compiler keeps there is lost. No vector
// register outputs.
__device__ __forceinline__ void gather_lds16(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(lds_base) : "memory");
}

// The same with a wave-uniform base address (in scalar registers) and a
// 32-bit per-lane byte offset: no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void gather_lds16_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(voff), "s"(sbase), "s"(lds_base) : "memory");
}

// One dword per active lane: lane i's 4 bytes at sbase + voff go to LDS
// address lds_base + 4 * i.
__device__ __forceinline__ void gather_lds4_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dword %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(voff), "s"(sbase), "s"(lds_base) : "memory");
}

template <int N_OUT>
__device__ __forceinline__ void wait_vm() {
  // s_waitcnt vmcnt(N_OUT), leaving expcnt and lgkmcnt unconstrained
  static_assert(N_OUT >= 0 && N_OUT < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N_OUT & 15) | ((N_OUT >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ------------------------------------------------------------------ misc
__host__ __device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

__device__ __forceinline__ int64_t visible(int32_t p, int32_t ratio, int64_t N) {
  if (p < 0) return 0;
  const int64_t n = (int64_t)(((uint32_t)p + 1u) / (uint32_t)ratio);   // 32-bit divide
  return n < N ? n : N;
}

// Kernel timer hook (defined in api.hip).
void timer_before(int kid, hipStream_t s);
void timer_after(int kid, hipStream_t s);

}  // namespace csa
