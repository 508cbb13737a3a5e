// append_row.h -- one token's row written into a paged-cache page in each cache
// format, shared by the append kernels and the layer front's fused append (both
// paths run these same functions, so they produce the same bytes).  The formats
// and their arithmetic are described at the top of append.hip; every function
// here takes the token's bf16 latent row (512) and RoPE key (64) by pointer (global
// memory or LDS) and a slot already checked against the pool.
#pragma once
#include "common.h"

namespace mla {

constexpr int kPageBf16 = kBlock * kRowBytesBf16;        // 73,728
constexpr int kPageInt8 = kBlock * 672;                  // 43,008
constexpr int kPageInt4 = kBlock * 480;                  // 30,720
constexpr int kPageInt4Sym = kBlock * 416;               // 26,624
constexpr int kPageInt8Tok = kBlock * 612;               // 39,168
constexpr int kPageInt4SymK4 = kBlock * 384;             // 24,576
// INT8 per channel over 32-token blocks (see append.hip)
constexpr int kPageInt8c = 59392;
constexpr int kI8cKeyCodes = 64 * 512, kI8cScales = kI8cKeyCodes + 64 * 64, kI8cKeyScales = kI8cScales + 2 * 512 * 4,
              kI8cOverflow = kI8cKeyScales + 64 * 8 * 4;
constexpr int kTBlk = 32;

__device__ __forceinline__ bool slot_ok(int64_t slot, int64_t num_pages) {
  return slot >= 0 && slot < num_pages * kBlock;
}

// Symmetric INT8 of `kG` consecutive bf16 values.
template <int kG>
__device__ __forceinline__ float quant_sym8(const uint16_t* x, int8_t* codes) {
  float v[kG];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kG; ++i) {
    v[i] = bf16_to_f32(x[i]);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const float scale = __fdiv_rn(amax, 127.0f);
#pragma unroll
  for (int i = 0; i < kG; ++i) {
    float q = 0.f;
    if (scale != 0.f) q = fminf(fmaxf(rintf(__fdiv_rn(v[i], scale)), -127.f), 127.f);
    codes[i] = (int8_t)(int)q;
  }
  return scale;
}

// e4m3 code of a finite y with |y| <= 448 (up to float rounding): nearest value
// of the e4m3 grid (bias 7, 3 mantissa bits, subnormal step 2^-9), ties to even,
// saturating at 448; the sign bit is y's.  Scaling by powers of two is exact, so
// rintf does the rounding: below 2^-6 in steps of 2^-9, above it in steps of
// 2^(e-3) with q = 1.mmm in eighths (q = 16 carries into the exponent field).
__device__ __forceinline__ uint8_t fp8_e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  int code;
  if (a < 0.015625f) {
    code = (int)rintf(a * 512.0f);
  } else {
    const int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;
    code = (e + 7) * 8 + (int)rintf(ldexpf(a, 3 - e)) - 8;
  }
  return (uint8_t)(min(code, 126) | (int)sign);
}

// e4m3 codes of `kG` consecutive bf16 values with scale = amax / 448.
template <int kG>
__device__ __forceinline__ float quant_fp8(const uint16_t* x, uint8_t* codes) {
  float v[kG];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kG; ++i) {
    v[i] = bf16_to_f32(x[i]);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const float scale = __fdiv_rn(amax, 448.0f);
#pragma unroll
  for (int i = 0; i < kG; ++i) codes[i] = scale != 0.f ? fp8_e4m3_code(__fdiv_rn(v[i], scale)) : (uint8_t)0;
  return scale;
}

// bf16: 16-byte chunk `chunk` of the row (0..63 latent, 64..71 RoPE key).
__device__ __forceinline__ void row_bf16(uint8_t* pool, int64_t slot, const uint16_t* c_row, const uint16_t* k_row,
                                         int chunk) {
  const u32x4 v = ld16(chunk < 64 ? c_row + chunk * 8 : k_row + (chunk - 64) * 8);
  st16(pool + (slot / kBlock) * kPageBf16 + (slot % kBlock) * kRowBytesBf16 + chunk * 16, v);
}

// INT8 per 32 channels: group `grp` of the row (0..15 latent, 16..23 RoPE key of 8).
__device__ __forceinline__ void row_int8(uint8_t* pool, int64_t slot, const uint16_t* c_row, const uint16_t* k_row,
                                         int grp) {
  uint8_t* page = pool + (slot / kBlock) * kPageInt8;
  const int off = (int)(slot % kBlock);
  if (grp < 16) {
    int8_t codes[32];
    const float s = quant_sym8<32>(c_row + grp * 32, codes);
    int8_t* dst = reinterpret_cast<int8_t*>(page + off * 576 + grp * 32);
#pragma unroll
    for (int i = 0; i < 32; ++i) dst[i] = codes[i];
    reinterpret_cast<float*>(page + 64 * 576)[off * 16 + grp] = s;
  } else {
    const int j = grp - 16;
    int8_t codes[8];
    const float s = quant_sym8<8>(k_row + j * 8, codes);
    int8_t* dst = reinterpret_cast<int8_t*>(page + off * 576 + 512 + j * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = codes[i];
    reinterpret_cast<float*>(page + 64 * 576 + 64 * 64)[off * 8 + j] = s;
  }
}

// Asymmetric INT4 per 32 channels, RoPE key INT8 per 8: group `grp` (0..23).
__device__ __forceinline__ void row_int4(uint8_t* pool, int64_t slot, const uint16_t* c_row, const uint16_t* k_row,
                                         int grp) {
  uint8_t* page = pool + (slot / kBlock) * kPageInt4;
  const int off = (int)(slot % kBlock);
  // page regions: nibbles [64][256] | rope codes [64][64] | scales [64][16] | zeros [64][16] | rope scales [64][8]
  uint8_t* nib = page;
  int8_t* rcodes = reinterpret_cast<int8_t*>(page + 64 * 256);
  float* scales = reinterpret_cast<float*>(page + 64 * 256 + 64 * 64);
  float* zeros = scales + 64 * 16;
  float* rscales = zeros + 64 * 16;
  if (grp < 16) {
    const uint16_t* x = c_row + grp * 32;
    float v[32];
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      v[i] = bf16_to_f32(x[i]);
      mn = fminf(mn, v[i]);
      mx = fmaxf(mx, v[i]);
    }
    const float scale = __fdiv_rn(mx - mn, 15.0f);
    uint8_t bytes[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      uint32_t q0 = 0, q1 = 0;
      if (scale != 0.f) {
        q0 = (uint32_t)(int)fminf(fmaxf(rintf(__fdiv_rn(v[2 * j] - mn, scale)), 0.f), 15.f);
        q1 = (uint32_t)(int)fminf(fmaxf(rintf(__fdiv_rn(v[2 * j + 1] - mn, scale)), 0.f), 15.f);
      }
      bytes[j] = (uint8_t)(q0 | (q1 << 4));
    }
    uint8_t* dst = nib + off * 256 + grp * 16;
#pragma unroll
    for (int j = 0; j < 16; ++j) dst[j] = bytes[j];
    scales[off * 16 + grp] = scale;
    zeros[off * 16 + grp] = mn;
  } else {
    const int j = grp - 16;
    int8_t codes[8];
    const float s = quant_sym8<8>(k_row + j * 8, codes);
#pragma unroll
    for (int i = 0; i < 8; ++i) rcodes[off * 64 + j * 8 + i] = codes[i];
    rscales[off * 8 + j] = s;
  }
}

// Symmetric INT4 per 32 channels; RoPE key INT8 per 8, or (kKey4) symmetric INT4
// per 8: group `grp` (0..23).
template <bool kKey4>
__device__ __forceinline__ void row_int4s(uint8_t* pool, int64_t slot, const uint16_t* c_row, const uint16_t* k_row,
                                          int grp) {
  uint8_t* page = pool + (slot / kBlock) * (kKey4 ? kPageInt4SymK4 : kPageInt4Sym);
  const int off = (int)(slot % kBlock);
  // page regions: nibbles [64][256] | rope codes [64][64] (kKey4: rope nibbles
  // [64][32]) | scales [64][16] | rope scales [64][8]
  uint8_t* nib = page;
  int8_t* rcodes = reinterpret_cast<int8_t*>(page + 64 * 256);
  float* scales = reinterpret_cast<float*>(page + 64 * 256 + 64 * (kKey4 ? 32 : 64));
  float* rscales = scales + 64 * 16;
  if (grp < 16) {
    const uint16_t* x = c_row + grp * 32;
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      v[i] = bf16_to_f32(x[i]);
      amax = fmaxf(amax, fabsf(v[i]));
    }
    const float scale = __fdiv_rn(amax, 7.0f);
    uint8_t bytes[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      int q0 = 0, q1 = 0;
      if (scale != 0.f) {
        q0 = (int)fminf(fmaxf(rintf(__fdiv_rn(v[2 * j], scale)), -7.f), 7.f);
        q1 = (int)fminf(fmaxf(rintf(__fdiv_rn(v[2 * j + 1], scale)), -7.f), 7.f);
      }
      bytes[j] = (uint8_t)((q0 + 8) | ((q1 + 8) << 4));
    }
    uint8_t* dst = nib + off * 256 + grp * 16;
#pragma unroll
    for (int j = 0; j < 16; ++j) dst[j] = bytes[j];
    scales[off * 16 + grp] = scale;
  } else if constexpr (kKey4) {
    const int j = grp - 16;
    const uint16_t* x = k_row + j * 8;
    float v[8];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = bf16_to_f32(x[i]);
      amax = fmaxf(amax, fabsf(v[i]));
    }
    const float scale = __fdiv_rn(amax, 7.0f);
    uint8_t* dst = page + 64 * 256 + off * 32 + j * 4;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      int q0 = 0, q1 = 0;
      if (scale != 0.f) {
        q0 = (int)fminf(fmaxf(rintf(__fdiv_rn(v[2 * b], scale)), -7.f), 7.f);
        q1 = (int)fminf(fmaxf(rintf(__fdiv_rn(v[2 * b + 1], scale)), -7.f), 7.f);
      }
      dst[b] = (uint8_t)((q0 + 8) | ((q1 + 8) << 4));
    }
    rscales[off * 8 + j] = scale;
  } else {
    const int j = grp - 16;
    int8_t codes[8];
    const float s = quant_sym8<8>(k_row + j * 8, codes);
#pragma unroll
    for (int i = 0; i < 8; ++i) rcodes[off * 64 + j * 8 + i] = codes[i];
    rscales[off * 8 + j] = s;
  }
}

// Per-token INT8 (kFp8 false) or e4m3 (kFp8) latent, RoPE key per 8 in the same
// code: one whole wave, lane l owning latent channels 8 l .. 8 l + 7 against the
// token's maximum (a wave reduction: the maximum is exact in any order), lanes
// 0-7 also RoPE-key group l.
template <bool kFp8>
__device__ __forceinline__ void row_tok(uint8_t* pool, int64_t slot, const uint16_t* c_row, const uint16_t* k_row,
                                        int lane) {
  uint8_t* page = pool + (slot / kBlock) * kPageInt8Tok;
  const int off = (int)(slot % kBlock);
  const uint16_t* x = c_row + 8 * lane;
  float v[8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = bf16_to_f32(x[i]);
    amax = fmaxf(amax, fabsf(v[i]));
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  const float scale = __fdiv_rn(amax, kFp8 ? 448.0f : 127.0f);
  uint8_t* dst = page + off * 576 + 8 * lane;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (kFp8) {
      dst[i] = scale != 0.f ? fp8_e4m3_code(__fdiv_rn(v[i], scale)) : (uint8_t)0;
    } else {
      float q = 0.f;
      if (scale != 0.f) q = fminf(fmaxf(rintf(__fdiv_rn(v[i], scale)), -127.f), 127.f);
      dst[i] = (uint8_t)(int8_t)(int)q;
    }
  }
  if (lane == 0) reinterpret_cast<float*>(page + 64 * 576)[off] = scale;
  if (lane < 8) {
    uint8_t rc[8];
    float s;
    if constexpr (kFp8) {
      s = quant_fp8<8>(k_row + lane * 8, rc);
    } else {
      int8_t c8[8];
      s = quant_sym8<8>(k_row + lane * 8, c8);
#pragma unroll
      for (int i = 0; i < 8; ++i) rc[i] = (uint8_t)c8[i];
    }
    uint8_t* rdst = page + off * 576 + 512 + lane * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) rdst[i] = rc[i];
    reinterpret_cast<float*>(page + 64 * 576 + 64 * 4)[off * 8 + lane] = s;
  }
}

// Per-channel INT8, the per-token part (one whole wave): lanes 0-7 quantise the
// RoPE key's 8-groups; the wave writes the latent row to its block's open
// storage unless `closes_here` (the same call closes the block, whose close then
// reads the row from the call's input).
__device__ __forceinline__ void row_int8c_tok(uint8_t* pool, int64_t slot, const uint16_t* c_row,
                                              const uint16_t* k_row, int lane, bool closes_here) {
  uint8_t* page = pool + (slot / kBlock) * (int64_t)kPageInt8c;
  const int off = (int)(slot % kBlock), blk = off / kTBlk, rr = off % kTBlk;
  if (lane < 8) {
    int8_t rc[8];
    const float s = quant_sym8<8>(k_row + lane * 8, rc);
    int8_t* rdst = reinterpret_cast<int8_t*>(page + kI8cKeyCodes + off * 64 + lane * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) rdst[i] = rc[i];
    reinterpret_cast<float*>(page + kI8cKeyScales)[off * 8 + lane] = s;
  }
  if (closes_here) return;
  const u32x4 v = ld16(c_row + 8 * lane);
  uint8_t* dst = lane < 32 ? page + (kTBlk * blk + rr) * 512 + 16 * lane : page + kI8cOverflow + rr * 512 + 16 * (lane - 32);
  st16(dst, v);
}

// Whether the call (slots[0..n)) also holds the last position of the block of
// the token at index tok (slot), i.e. closes it: index tok + 31 - row.
__device__ __forceinline__ bool int8c_closes_here(const int64_t* slots, int n, int64_t tok, int64_t slot) {
  const int rr = (int)(slot % kTBlk);
  const int64_t jc = tok + (kTBlk - 1 - rr);
  return jc < n && slots[jc] == slot + (kTBlk - 1 - rr);
}

// One token's append by a work-group of 256 threads (thread tid), the row in
// c_row / k_row: the same function, thread for thread, as the append kernels.
// Formats 0-6 (the per-channel INT8 format's append has to close blocks across
// tokens and runs as its own launches).
__device__ __forceinline__ void append_row_wg(int cache_dtype, uint8_t* pool, int64_t slot, const uint16_t* c_row,
                                              const uint16_t* k_row, int tid) {
  switch (cache_dtype) {
    case 0: if (tid < 72) row_bf16(pool, slot, c_row, k_row, tid); break;
    case 1: if (tid < 24) row_int8(pool, slot, c_row, k_row, tid); break;
    case 2: if (tid < 24) row_int4(pool, slot, c_row, k_row, tid); break;
    case 3: if (tid < 24) row_int4s<false>(pool, slot, c_row, k_row, tid); break;
    case 4: if (tid < 64) row_tok<false>(pool, slot, c_row, k_row, tid); break;
    case 5: if (tid < 64) row_tok<true>(pool, slot, c_row, k_row, tid); break;
    case 6: if (tid < 24) row_int4s<true>(pool, slot, c_row, k_row, tid); break;
    default: break;
  }
}

}  // namespace mla
