// Device-side helpers shared by the CSA2 gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(8))) int i32x8;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Order-preserving map float -> u32 (larger float -> larger key); -0 maps like +0.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// max(x, 0) in one integer max on the bits (a negative float, -0 included, is a negative
// int32).  fmaxf (and its equivalents) costs two v_max_f32 here: the compiler first
// canonicalizes a value it cannot prove canonical, such as an MFMA result.  Differs from
// fmaxf only for NaN with the sign bit clear, which stays NaN.
__device__ __forceinline__ float relu_f32(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// The inverse of float_key: the float whose key is k (key 0x80000000 -> +0).
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// E8M0 scale byte -> fp32 2^(b - 127) (byte 0 -> the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return __uint_as_float(b ? (b << 23) : 0x00400000u);
}

// 8 E2M1 codes (one dword, low nibble first) times an E8M0 scale -> 8 bf16 (exact).
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w, float scale) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// 8 E2M1 codes times an E8M0 scale -> 4 packed f16 pairs (channel 2k low, 2k+1 high).
// Exact while the scale keeps every value in fp16 range (scale byte 104..140).
__device__ __forceinline__ void fp4x8_to_f16_pairs(uint32_t w, float scale, uint32_t out[4]) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 0));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 1));
  out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 2));
  out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 3));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

__device__ __forceinline__ u32x4 ld_global_16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// 16-byte streaming load (non-temporal: data read once, not kept in the caches for reuse)
__device__ __forceinline__ u32x4 ld_global_16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// 16-byte load from an address held as an integer, kept in the global address space (a
// generic pointer would become a flat load, which also counts against LDS waits).
__device__ __forceinline__ u32x4 ld_global_16_addr(uint64_t a) {
  return *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(a);
}

// Wait until every vector memory access issued so far has completed (the counter covers
// loads and stores on this architecture).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (Hillis-Steele within
// each 16-lane row by row_shr 1, 2, 4, 8, then row_bcast 15 / 31 carry the row totals).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Inclusive prefix sum within each 16-lane row of the wave (the first four steps above).
__device__ __forceinline__ uint32_t row16_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  return v;
}

// Lane 15 of each 16-lane row, broadcast to the row (DPP row_newbcast:15).
__device__ __forceinline__ uint32_t row16_last(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x15f, 0xf, 0xf, false);
}

// max(a - b, 0) for unsigned values, written without a comparison-guarded subtraction:
// this compiler has been seen to hoist the subtraction of `a > b ? f(a - b) : 0` with a
// no-wrap flag and then treat b <= a as known elsewhere (dropping a later min(b, a)).
__device__ __forceinline__ uint32_t sub_sat_u32(uint32_t a, uint32_t b) { return a - min(a, b); }

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

}  // namespace csa2
