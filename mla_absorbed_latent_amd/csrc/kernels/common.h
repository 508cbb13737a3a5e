// common.h -- shared device helpers for the gfx950 kernels (CDNA4 only).
//
// Vector types, MFMA and LDS-transpose wrappers, bf16/fp16 conversions, and the
// cache page geometry.  Lane layouts of the matrix instructions used here
// (checked on gfx950 with known matrices):
//   v_mfma_f32_32x32x16_{f16,bf16}: lane l holds A[m = l%32][k = 8(l/32)+0..7],
//       B[k = 8(l/32)+0..7][n = l%32]; D register r is
//       D[m = 8(r/4) + 4(l/32) + r%4][n = l%32], r = 0..15.
//   v_mfma_f32_16x16x32_f16: A[m = l%16][k = 8(l/16)+0..7], B[k = 8(l/16)+0..7][n = l%16];
//       D register r is D[m = 4(l/16) + r][n = l%16], r = 0..3.
//   v_mfma_f32_16x16x16_f16: as above with 4 k values per lane (k = 4(l/16)+0..3).
//   ds_read_b64_tr_b16: within each group of 16 lanes, lane i slot s receives
//       element i%4 of the 8-byte chunk addressed by group lane 4s + i/4.  If group
//       lane j addresses row r0 + j/4, columns c0 + 4(j%4) .. +3 of a row-major
//       16-bit matrix, lane i receives column c0 + i of rows r0 .. r0+3: a
//       transposed 4 x 16 read.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) char lds_char;

constexpr int kBlock = 64;      // tokens per page
constexpr int kDc = 512;        // latent width
constexpr int kDr = 64;         // RoPE key width
constexpr int kDk = 576;        // score width (latent + RoPE key)
constexpr int kDn = 128;        // qk_nope / v head width
constexpr int kRowBytesBf16 = kDk * 2;   // 1,152 B per cached bf16 token

__device__ __forceinline__ floatx16 mfma32x32x16(half8 a, half8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx16 mfma32x32x16_bf16(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16x16x32(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16x16x16(half4 a, half4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Transposed 4x16 LDS read (see header); `byte_off` is this lane's chunk address.
__device__ __forceinline__ half4 lds_read_tr(const void* lds_base, uint32_t byte_off) {
  short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v*)((lds_char*)lds_base + byte_off));
  return __builtin_bit_cast(half4, v);
}

// Two bf16 values (low, high) -> two fp16 values.  bf16 carries 8 significant
// bits, so every bf16 in the fp16 range is exact in fp16 and round-toward-zero
// changes nothing; values below 2^-17 lose low bits, values beyond 65504
// saturate to +-65504.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v) {
  float lo = __uint_as_float(v << 16);
  float hi = __uint_as_float(v & 0xffff0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  u32x4 r;
  r[0] = bf16x2_to_f16x2(v[0]);
  r[1] = bf16x2_to_f16x2(v[1]);
  r[2] = bf16x2_to_f16x2(v[2]);
  r[3] = bf16x2_to_f16x2(v[3]);
  return r;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);  // round to nearest even
}

// 16-byte global loads / stores.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Maximum over lanes l and l ^ 32, within the VALU: v_permlane32_swap of x with
// itself gives the lower half-wave in both halves of its first result and the
// upper half-wave in both halves of its second.
__device__ __forceinline__ float max_xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
}

// Maximum over lanes l, l ^ 16, l ^ 32 and l ^ 48, within the VALU: each
// v_permlane*_swap of x with itself gives, in its two results, the two lanes
// of every pair (l, l ^ 16) or (l, l ^ 32).
__device__ __forceinline__ float max_xor16_32(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  u = __builtin_bit_cast(uint32_t, fmaxf(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1])));
  const auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)b[0]), __builtin_bit_cast(float, (uint32_t)b[1]));
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

}  // namespace mla
