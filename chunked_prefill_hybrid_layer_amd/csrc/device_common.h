// Device helpers shared by the gfx950 kernels: bf16 packing, MFMA fragment
// types, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hb_internal.h"

namespace hb {

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).  Direct-to-LDS
// loads (global_load_lds) count in vmcnt; the compiler does not reliably wait
// for them before a barrier, so kernels that stage tiles that way wait
// explicitly before the barrier that publishes a tile.
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
// s_waitcnt with only the LDS/scalar counter constrained (lgkmcnt = 0)
#define WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4))

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streaming loads (data read once): the nontemporal hint keeps them from
// displacing reused data in the caches.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_stream8(const void* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t load_stream4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// FP8 e4m3 (OCP e4m3fn) KV storage.  The conversion instruction rounds to
// nearest even but turns magnitudes past 448's rounding range into NaN, so
// values are clamped to +-448 first (saturating codes).
__device__ __forceinline__ float clamp448(float x) { return fminf(fmaxf(x, -448.0f), 448.0f); }
// four floats -> four codes, byte i holding value i
__device__ __forceinline__ uint32_t pack4fp8(float a, float b, float c, float d) {
  const uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), lo, true);
}
__device__ __forceinline__ uint8_t fp8_code(float a) {
  return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), 0.0f, 0, false) & 0xffu);
}
// two codes (the low or high half of w) -> two bf16 in one word, exactly
// (every e4m3 value is a bf16 value)
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
__device__ __forceinline__ uint2 fp8x4_bf16x4(uint32_t w) {
  return make_uint2(fp8x2_bf16x2<false>(w), fp8x2_bf16x2<true>(w));
}
__device__ __forceinline__ uint4 fp8x8_bf16x8(uint2 w) {
  return make_uint4(fp8x2_bf16x2<false>(w.x), fp8x2_bf16x2<true>(w.x), fp8x2_bf16x2<false>(w.y),
                    fp8x2_bf16x2<true>(w.y));
}

// float -> bf16, round to nearest even, NaN kept (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// two floats -> packed bf16 pair (lo in bits 0..15), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// FP8 e4m3 x e4m3 MFMA (gfx950 f8f6f4 family, format 0 for both operands,
// unit E8M0 block scales): D[16][16] += A[16][128] B^T.  Lane l holds row
// (or column) l % 16 and 32 of the 128 K positions; which 32 does not matter
// as long as A and B use the same assignment (checked on the device).
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma16x16x128_f8(const i32x8& a, const i32x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ i32x8 cat_i32x8(const uint4& lo, const uint4& hi) {
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// LDS destination of a direct-to-LDS load (global_load_lds_dwordx4): the
// wave's 64 lanes land at consecutive 16-byte chunks from this address.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

// The value of lane l ^ 32 (xor32) or l ^ 16 (xor16), through gfx950's
// v_permlane32_swap / v_permlane16_swap: two VALU instructions and a select,
// where a shuffle goes through the LDS crossbar (ds_bpermute) and its latency.
// Each swap takes two copies of x and returns them with the upper half (of
// the wave, or of each 32-lane row pair) of the first exchanged with the
// lower half of the second; the partner's value is in the copy the lane's
// own half did not keep.
__device__ __forceinline__ float xor32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 16) ? r[0] : r[1]);
}

__device__ __forceinline__ float wave_sum(float v) {
  v += xor32(v);
  v += xor16(v);
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, xor32(v));
  v = fmaxf(v, xor16(v));
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace hb
