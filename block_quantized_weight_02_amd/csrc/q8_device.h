// q8_device.h -- device helpers shared by the library's kernel sources:
// weight-stream loads, byte converts, the packed scale position, the block
// quantizer's arithmetic and the MFMA operand types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q8_internal.h"

namespace q8 {
namespace dev {

__device__ __forceinline__ float bf16_lo(uint32_t pair) {  // element 2p
  return __uint_as_float(pair << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t pair) {  // element 2p+1
  return __uint_as_float(pair & 0xffff0000u);
}

// Loads of the weight stream.  The values are loaded non-temporal (read once
// per call, they must not displace the activation or the carries from the
// caches); the scales, an eighth of the bytes, with the default policy, which
// measured faster on MI355X (m=1, K=4096, N=14336: 11.9 against 12.2 us with
// non-temporal scales; values without it: 13.4 us).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_stream16(const void *p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream8(const void *p) {
  const u32x2_t v = __builtin_nontemporal_load(static_cast<const u32x2_t *>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ float ld_scale4f(const float *p) { return *p; }
__device__ __forceinline__ float4 ld_scale16f(const float4 *p) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  const f32x4v v = *reinterpret_cast<const f32x4v *>(p);
  return make_float4(v.x, v.y, v.z, v.w);
}

// Buffer loads of the weight stream: a wave-uniform resource (base address
// and byte extent, in scalar registers), a 32-bit lane offset and a uniform
// block offset -- no per-lane 64-bit addresses, and loads outside the extent
// return zero.  Cache policy as above: values non-temporal, scales default.
typedef __amdgpu_buffer_rsrc_t buf_t;
constexpr int kBufNT = 2;                 // the nt cache-policy bit
constexpr int kBufFlags = 0x00020000;     // resource word 3: 32-bit data format
__device__ __forceinline__ buf_t make_buf(const void *base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           kBufFlags);
}
__device__ __forceinline__ uint4 buf_ld16(buf_t r, unsigned voff, unsigned soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kBufNT);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float buf_ld4f(buf_t r, unsigned voff, unsigned soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// 16-byte stores and loads with the cache-policy bits of a system-scope
// relaxed atomic (sc0 sc1): written through to memory and read from it, past
// the per-XCD L2s, so a workgroup on another XCD sees them once the writer's
// stores have completed.
constexpr int kBufSys = 17;
__device__ __forceinline__ void buf_st16_sys(buf_t r, unsigned voff, float4 v) {
  const u32x4_t d = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                     __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(d, r, voff, 0, kBufSys);
}
__device__ __forceinline__ float4 buf_ld16_sys(buf_t r, unsigned voff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kBufSys);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                     __uint_as_float(v.w));
}

// The four signed bytes of a dword as fp32 (exact); byte j is k = 4d + j.
__device__ __forceinline__ void i8x4_to_f32(uint32_t v, float *f) {
  f[0] = (float)(int8_t)(v);
  f[1] = (float)(int8_t)(v >> 8);
  f[2] = (float)(int8_t)(v >> 16);
  f[3] = (float)((int32_t)v >> 24);
}

// Position of column c's scale inside a chunk's 64-float scale row: the four
// columns c = i + 16g (g = 0..3) of one lane index i sit together, so an MFMA
// lane reads its four column groups' scales as one 16-byte load and a VALU
// lane (column c) one dword.
__device__ __forceinline__ int scale_pos(int c) { return ((c & 15) << 2) | (c >> 4); }


// The quantizer of an activation block (also the product's output
// quantizer): scale from the block's amax, then one code per value.  Both
// divisions are fp32 divisions rounded correctly (the library is built with
// -fhip-fp32-correctly-rounded-divide-sqrt): the same value as an fp64
// quotient of the fp32 operands rounded once to fp32, since 53 >= 2 * 24 + 2
// bits make that double rounding innocuous.
__device__ __forceinline__ float q8_quot(float a, float b) { return a / b; }

__device__ __forceinline__ float q8_scale_of(float amax) { return q8_quot(amax, 127.0f); }

__device__ __forceinline__ int8_t q8_code_of(float v, float d) {
  if (d == 0.0f) return 0;
  const float rq = roundf(q8_quot(v, d));   // ties away from zero
  return (int8_t)(int)fminf(fmaxf(rq, -127.0f), 127.0f);
}

// MFMA operand and result types.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;

// Eight int8 -> eight bf16 (exact: |q| <= 127 needs 8 significant bits).
__device__ __forceinline__ bf16x8_t i8x8_to_bf16(uint2 v) {
  float f[8];
  i8x4_to_f32(v.x, f);
  i8x4_to_f32(v.y, f + 4);
  uint32_t p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    p[e] = __builtin_amdgcn_perm(__float_as_uint(f[2 * e + 1]), __float_as_uint(f[2 * e]),
                                 0x07060302u);
  return __builtin_bit_cast(bf16x8_t, make_uint4(p[0], p[1], p[2], p[3]));
}

// Copies words of a weight stage into fresh registers before lane swaps
// (v_permlane16/32_swap overwrite both of their operands).  Without the copy
// the register allocator of a two-stage loop can tie the swaps to registers
// that the next stage's load (still in flight) is given, and the loop then
// waits for that load too; the copy is a move the compiler cannot fold.
template <int N, int D>
__device__ __forceinline__ void opaque_copy(uint32_t (&r)[N][D]) {
#pragma unroll
  for (int a = 0; a < N; ++a)
#pragma unroll
    for (int d = 0; d < D; ++d) asm volatile("v_mov_b32 %0, %1" : "=v"(r[a][d]) : "v"(r[a][d]));
}

}  // namespace dev
}  // namespace q8
