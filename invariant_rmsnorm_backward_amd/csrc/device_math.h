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

__device__ __forceinline__ void unpack4(const uint2& v, float (&f)[4]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
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

// Streaming (non-temporal) 16-byte global accesses for data touched once:
// the loads and stores carry the nt cache policy, so a pass over hundreds of
// MB does not evict what other kernels keep in L2 and the Infinity Cache.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 load8_stream(const void* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void store16_stream(void* p, const uint4& v) {
  const u32x4_t u = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(u, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void store_f4_stream(float* p, float a, float b, float c, float d) {
  const u32x4_t u = {__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
  __builtin_nontemporal_store(u, reinterpret_cast<u32x4_t*>(p));
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

// Wavefront sum with DPP lane moves inside each 16-lane row, then the four
// row sums combined in a fixed order from scalar reads.  Every lane returns
// the same bits: within a row each step adds a lane's value to its partner's
// (a+b == b+a), and the final combination is computed from uniform values.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = v + dpp_move<0xB1>(v);    // quad_perm [1,0,3,2]: pairs
  v = v + dpp_move<0x4E>(v);    // quad_perm [2,3,0,1]: quads
  v = v + dpp_move<0x141>(v);   // row_half_mirror: 8 lanes
  v = v + dpp_move<0x140>(v);   // row_mirror: 16 lanes
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// The in-block stream tree of the canonical order: (q0+q1)+(q2+q3).
__device__ __forceinline__ float stream_tree4(float q0, float q1, float q2, float q3) {
  return (q0 + q1) + (q2 + q3);
}

}  // namespace rbi
