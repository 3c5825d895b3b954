// device_math.h -- gfx950 device helpers: bf16 <-> FP32, 16-byte vectors,
// and wavefront (64-lane) butterfly reductions.
//
// Every function here is deterministic: the same inputs give the same bits
// in every lane, every wave and every launch.  The library is compiled with
// -ffp-contract=off, so a*b+c is two rounded operations unless fmaf is
// written out.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rbi {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 is the upper half of binary32: widening is a shift (exact).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Two FP32 values -> two bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

// Element e (0..7) of a 16-byte vector of 8 bf16.
__device__ __forceinline__ float bf16x8_get(const uint4& v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  uint4 r;
  r.x = pack_bf16x2(f[0], f[1]);
  r.y = pack_bf16x2(f[2], f[3]);
  r.z = pack_bf16x2(f[4], f[5]);
  r.w = pack_bf16x2(f[6], f[7]);
  return r;
}

__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void store16(void* p, const uint4& v) {
  *reinterpret_cast<uint4*>(p) = v;
}
__device__ __forceinline__ void store_f4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// Register "laundering": an empty asm that claims to modify the value.  Used
// between the two passes over a row so the compiler re-derives FP32 values
// from the packed bf16 registers instead of keeping 2x as many registers
// live across the row reduction.  Emits no instruction.
__device__ __forceinline__ void launder(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}
// Compiler-only memory fence: values read from LDS before it are read again
// after it (no instruction, no hardware wait).
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Sum over groups of G consecutive lanes (G a power of two, <= 64) by an xor
// butterfly.  At each level lane i adds the value of lane i^k; since a+b and
// b+a are the same FP32 value, every lane of a group ends with the same bits.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int k = G / 2; k >= 1; k >>= 1) v = v + __shfl_xor(v, k, 64);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

// The in-block stream tree of the canonical order: ((q0+q1)+(q2+q3))+((q4+q5)+(q6+q7)).
__device__ __forceinline__ float stream_tree8(const float (&q)[8]) {
  return ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
}

}  // namespace rbi
