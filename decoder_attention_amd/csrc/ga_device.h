// Device-side helpers shared by the Gemma attention kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ga {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// Two floats -> packed bf16 pair (low = a), round to nearest even: one
// v_cvt_pk_bf16_f32 (converting the halves separately and merging them costs
// four instructions).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// LDS pointer cast for the transpose-read builtin.
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i%4
// of the 8-byte chunks addressed by lanes 4e + i/4, e = 0..3.  Pointing lane j
// of a group at row (r0 + j/4), column (c0 + 4*(j%4)) of a row-major bf16 tile
// therefore gives lane i the four rows r0..r0+3 at column c0 + i.
// Direct-to-LDS copy, buffer form: every lane copies Bytes (4 or 16) from
// rsrc base + voff to lds + Bytes * lane, with cache-policy bits Aux.  Unlike
// the global-segment form, the compiler counts this copy on the vector-memory
// counter only, so the LDS reads issued around it keep partial waits instead
// of waiting for every outstanding LDS read.  Offsets past the resource's
// byte range read zeros.
// (The builtin takes its size and policy only as literal constants.)
template <int Bytes = 16, int Aux = 0>
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, void* lds) {
  auto* dst = (__attribute__((address_space(3))) void*)(lds);
  static_assert((Bytes == 16 || Bytes == 4) && (Aux == 0 || Aux == 2), "copy size / policy");
  if constexpr (Bytes == 16 && Aux == 0) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff, 0, 0, 0);
  else if constexpr (Bytes == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff, 0, 0, 2);
  else if constexpr (Aux == 0) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 4, voff, 0, 0, 0);
  else __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 4, voff, 0, 0, 2);
}

// Rotary helpers shared by the QK prologue (its per-token tables) and the
// attention kernel's in-register query rotation, so that both turn a query
// by exactly the same arithmetic.
//
// Frequency of rotate-half pair i in revolutions per position:
// c0 * w1^i with w1 = theta^(-2/r) and c0 = 1 / (2 pi pos_div), by one fixed
// chain of fp64 products: i = 16a + 8b + e gives ((c0 * w8^b) * w16^a) * w1^e,
// multiplied out in that order (w2 = w1 w1, w4 = w2 w2, w8 = w4 w4,
// w16 = w8 w8).  A few fp64 ulps from the exact power.
__device__ __forceinline__ double rotary_rev_freq(int32_t i, double w1, double c0) {
  const double w2 = w1 * w1, w4 = w2 * w2, w8 = w4 * w4, w16 = w8 * w8;
  double f = ((i >> 3) & 1) ? c0 * w8 : c0;
  for (int32_t a = 0; a < (i >> 4); ++a) f *= w16;
  for (int32_t e = 0; e < (i & 7); ++e) f *= w1;
  return f;
}
// (cos, sin) at position p for frequency f (revolutions per position): the
// fractional part of p * f taken in fp64, then the hardware fp32 cosine and
// sine, which take revolutions (measured on gfx950 against fp64: within
// 1.3e-7).
__device__ __forceinline__ float2 rotary_cos_sin(double p, double f) {
  const float r = static_cast<float>(__builtin_amdgcn_fract(p * f));
  return make_float2(__builtin_amdgcn_cosf(r), __builtin_amdgcn_sinf(r));
}
// One rotated element: x cos + partner * s, with s = -sin for the lower half
// of a pair (partner = upper) and +sin for the upper half (partner = lower).
__device__ __forceinline__ float rotary_turn(float x, float partner, float c, float s) {
  return __builtin_fmaf(x, c, partner * s);
}

// Workgroup barrier for LDS traffic that leaves direct-to-LDS copies in
// flight.  __syncthreads() carries a workgroup fence, and a direct-to-LDS copy
// counts as an LDS write on the vector-memory counter, so the compiler puts
// s_waitcnt vmcnt(0) before every such barrier: each barrier inside a
// copy-ahead loop would wait for the tiles still meant to be in flight.  Here
// the wave waits only for its own LDS reads and writes (lgkmcnt(0)), so after
// the barrier every wave's LDS stores are visible and every wave's reads of
// the previous contents are done.  Callers wait for the copies they need
// (vmcnt) before it.  The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // gfx9 encoding: lgkmcnt(0); vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Debug build (compiled with GA_LDS_POISON=1): every LDS array of a kernel
// starts filled with all-ones bytes, which is a NaN in bf16, fp16, fp32 and
// fp64, so reading a location the kernel has not written turns an output
// non-finite.  (For int8 codes the byte 0xFF is the valid code -1; those
// tiles are covered through their fp32 scales, copied alongside.)  Called
// by every thread of the workgroup before anything else touches the LDS.
#ifndef GA_LDS_POISON
#define GA_LDS_POISON 0
#endif
template <typename... A>
__device__ __forceinline__ void lds_poison(A&... arrs) {
  if constexpr (GA_LDS_POISON != 0) {
    auto fill = [](void* base, uint32_t bytes) {
      uint32_t* w = static_cast<uint32_t*>(base);
      for (uint32_t i = threadIdx.x; i < bytes / 4; i += blockDim.x) w[i] = 0xffffffffu;
    };
    (fill(static_cast<void*>(&arrs), static_cast<uint32_t>(sizeof(arrs))), ...);
    __syncthreads();
  }
}

// Buffer resource over nbytes from base (raw addressing, 32-bit offsets).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int32_t>(nbytes), 0x00020000);
}

__device__ __forceinline__ i16x4 lds_read_tr16(const void* lds_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_addr));
}

typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i32 lds_v2i32;

// ds_read_b64_tr_b8: within each 16-lane group, lane i receives byte i%8 of
// the 8-byte chunks addressed by lanes 2e + i/8, e = 0..7, as its bytes e.
// Pointing lane j of a group at row key(j/2), column (c0 + 8*(j%2)) of a
// row-major byte tile therefore gives lane i the eight rows key(0..7) at
// column c0 + i.
__device__ __forceinline__ v2i32 lds_read_tr8(const void* lds_addr) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)(lds_addr));
}

// Two signed bytes (B, B+1) of w as a bf16 pair.  Integers up to 128 in
// magnitude have 8 significant bits, so their fp32 value truncates to bf16
// exactly (the high half).
template <int B>
__device__ __forceinline__ uint32_t i8pair_to_bf16x2(uint32_t w) {
  const float lo = static_cast<float>(static_cast<int32_t>(w << (24 - 8 * B)) >> 24);
  const float hi = static_cast<float>(static_cast<int32_t>(w << (16 - 8 * B)) >> 24);
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Eight signed bytes (w0 bytes 0-3, w1 bytes 0-3) as eight bf16 values.
__device__ __forceinline__ bf16x8 i8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return __builtin_bit_cast(bf16x8, u32x4{i8pair_to_bf16x2<0>(w0), i8pair_to_bf16x2<2>(w0), i8pair_to_bf16x2<0>(w1),
                                          i8pair_to_bf16x2<2>(w1)});
}

// int8 codes as offset fp16.  Flipping a code's sign bit gives u = c + 128
// in [0, 255]; the fp16 bit pattern 0x64 : u is 1024 + u = 1152 + c exactly
// (exponent 2^10, u in the low mantissa bits), so one byte permute per two
// codes converts them (a product against these values carries an extra
// 1152 * sum of the other operand, which the caller removes).
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
constexpr float kI8Offset = 1152.f;
__device__ __forceinline__ uint32_t i8pair_to_f16x2_off(uint32_t flipped, uint32_t sel) {
  return __builtin_amdgcn_perm(0x64646464u, flipped, sel);
}
// Eight codes (w0 bytes 0-3, w1 bytes 0-3) as eight offset fp16 values.
__device__ __forceinline__ f16x8 i8x8_to_f16x8_off(uint32_t w0, uint32_t w1) {
  const uint32_t a = w0 ^ 0x80808080u, b = w1 ^ 0x80808080u;
  return __builtin_bit_cast(f16x8, u32x4{i8pair_to_f16x2_off(a, 0x04010400u), i8pair_to_f16x2_off(a, 0x04030402u),
                                         i8pair_to_f16x2_off(b, 0x04010400u), i8pair_to_f16x2_off(b, 0x04030402u)});
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2));
}

__device__ __forceinline__ float wave_max_xor32(float v) {
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float wave_sum_xor32(float v) {
  return v + __shfl_xor(v, 32, 64);
}

}  // namespace ga
