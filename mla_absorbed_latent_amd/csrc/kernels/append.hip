// append.hip -- write new tokens' latent rows into the paged cache, quantising
// on the way in for the INT8 / INT4 formats.
//
// Only the 512-wide latent and the 64-wide RoPE key are cached
// ("DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界" §2.4, §4.1).  The quantised
// formats follow "DeepSeek-V2-Lite MLA 吸收式 KV 缓存优化 — 完整实验报告" §3.2 / §4.1
// (INT8 with 32-element blocks, asymmetric INT4 with 32-element blocks, RoPE key
// INT8 with 8-element blocks).  Each block is one token's consecutive channels,
// so a token is quantised by itself.  Arithmetic is IEEE fp32 with correctly
// rounded division and round-half-even, so codes and scales are reproducible
// bit for bit:
//   INT8: scale = amax / 127, code = clamp(rint(x / scale), -127, 127); amax 0 -> 0.
//   INT4: zero = min, scale = (max - min) / 15, q = clamp(rint((x - min) / scale), 0, 15);
//         scale 0 -> q 0; two codes a byte, element 2j in the low nibble.
//   INT8 per token (a variant the report does not measure): the INT8 rule with one
//         group of all 512 latent channels; RoPE key as INT8.
//   INT4 symmetric (a variant the report does not measure): scale = amax / 7,
//         q = clamp(rint(x / scale), -7, 7), stored as the nibble q + 8; amax 0 -> 8.
//   INT8 per channel over 32-token blocks: see append_int8c_close below (a block
//         is quantised when its 32nd token arrives).
//
// One thread per 16-byte chunk (bf16) or per quantisation group; slots outside
// [0, num_pages * 64) are skipped.
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int kPageBf16 = kBlock * kRowBytesBf16;        // 73,728
constexpr int kPageInt8 = kBlock * 672;                  // 43,008
constexpr int kPageInt4 = kBlock * 480;                  // 30,720
constexpr int kPageInt4Sym = kBlock * 416;               // 26,624
constexpr int kPageInt8Tok = kBlock * 612;               // 39,168
constexpr int kPageInt4SymK4 = kBlock * 384;             // 24,576

__device__ __forceinline__ bool slot_ok(int64_t slot, int64_t num_pages) {
  return slot >= 0 && slot < num_pages * kBlock;
}

__global__ __launch_bounds__(256) void append_bf16(uint8_t* pool, int64_t num_pages, const uint16_t* c_kv,
                                                   const uint16_t* k_pe, const int64_t* slots, int n) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t tok = gid / 72;
  const int chunk = (int)(gid % 72);
  if (tok >= n) return;
  // Both loads are issued before either is used (one memory round trip).
  const uint16_t* src = chunk < 64 ? c_kv + tok * kDc + chunk * 8 : k_pe + tok * kDr + (chunk - 64) * 8;
  const u32x4 v = ld16(src);
  const int64_t slot = slots[tok];
  if (!slot_ok(slot, num_pages)) return;
  uint8_t* dst = pool + (slot / kBlock) * kPageBf16 + (slot % kBlock) * kRowBytesBf16 + chunk * 16;
  st16(dst, v);
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

// 24 groups a token: 16 latent groups of 32, then 8 RoPE-key groups of 8.
__global__ __launch_bounds__(256) void append_int8(uint8_t* pool, int64_t num_pages, const uint16_t* c_kv,
                                                   const uint16_t* k_pe, const int64_t* slots, int n) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t tok = gid / 24;
  const int grp = (int)(gid % 24);
  if (tok >= n) return;
  const int64_t slot = slots[tok];
  if (!slot_ok(slot, num_pages)) return;
  uint8_t* page = pool + (slot / kBlock) * kPageInt8;
  const int off = (int)(slot % kBlock);
  if (grp < 16) {
    int8_t codes[32];
    const float s = quant_sym8<32>(c_kv + tok * kDc + grp * 32, codes);
    int8_t* dst = reinterpret_cast<int8_t*>(page + off * 576 + grp * 32);
#pragma unroll
    for (int i = 0; i < 32; ++i) dst[i] = codes[i];
    reinterpret_cast<float*>(page + 64 * 576)[off * 16 + grp] = s;
  } else {
    const int j = grp - 16;
    int8_t codes[8];
    const float s = quant_sym8<8>(k_pe + tok * kDr + j * 8, codes);
    int8_t* dst = reinterpret_cast<int8_t*>(page + off * 576 + 512 + j * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = codes[i];
    reinterpret_cast<float*>(page + 64 * 576 + 64 * 64)[off * 8 + j] = s;
  }
}

// 24 groups a token: 16 asymmetric INT4 latent groups of 32, then 8 INT8 RoPE-key groups.
__global__ __launch_bounds__(256) void append_int4(uint8_t* pool, int64_t num_pages, const uint16_t* c_kv,
                                                   const uint16_t* k_pe, const int64_t* slots, int n) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t tok = gid / 24;
  const int grp = (int)(gid % 24);
  if (tok >= n) return;
  const int64_t slot = slots[tok];
  if (!slot_ok(slot, num_pages)) return;
  uint8_t* page = pool + (slot / kBlock) * kPageInt4;
  const int off = (int)(slot % kBlock);
  // page regions: nibbles [64][256] | rope codes [64][64] | scales [64][16] | zeros [64][16] | rope scales [64][8]
  uint8_t* nib = page;
  int8_t* rcodes = reinterpret_cast<int8_t*>(page + 64 * 256);
  float* scales = reinterpret_cast<float*>(page + 64 * 256 + 64 * 64);
  float* zeros = scales + 64 * 16;
  float* rscales = zeros + 64 * 16;
  if (grp < 16) {
    const uint16_t* x = c_kv + tok * kDc + grp * 32;
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
    const float s = quant_sym8<8>(k_pe + tok * kDr + j * 8, codes);
#pragma unroll
    for (int i = 0; i < 8; ++i) rcodes[off * 64 + j * 8 + i] = codes[i];
    rscales[off * 8 + j] = s;
  }
}

// 24 groups a token: 16 symmetric INT4 latent groups of 32, then 8 INT8 RoPE-key groups.
// kKey4: the RoPE key by the same symmetric INT4 rule in groups of 8.
template <bool kKey4>
__global__ __launch_bounds__(256) void append_int4s(uint8_t* pool, int64_t num_pages, const uint16_t* c_kv,
                                                    const uint16_t* k_pe, const int64_t* slots, int n) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t tok = gid / 24;
  const int grp = (int)(gid % 24);
  if (tok >= n) return;
  const int64_t slot = slots[tok];
  if (!slot_ok(slot, num_pages)) return;
  uint8_t* page = pool + (slot / kBlock) * (kKey4 ? kPageInt4SymK4 : kPageInt4Sym);
  const int off = (int)(slot % kBlock);
  // page regions: nibbles [64][256] | rope codes [64][64] (kKey4: rope nibbles
  // [64][32]) | scales [64][16] | rope scales [64][8]
  uint8_t* nib = page;
  int8_t* rcodes = reinterpret_cast<int8_t*>(page + 64 * 256);
  float* scales = reinterpret_cast<float*>(page + 64 * 256 + 64 * (kKey4 ? 32 : 64));
  float* rscales = scales + 64 * 16;
  if (grp < 16) {
    const uint16_t* x = c_kv + tok * kDc + grp * 32;
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
    const uint16_t* x = k_pe + tok * kDr + j * 8;
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
    const float s = quant_sym8<8>(k_pe + tok * kDr + j * 8, codes);
#pragma unroll
    for (int i = 0; i < 8; ++i) rcodes[off * 64 + j * 8 + i] = codes[i];
    rscales[off * 8 + j] = s;
  }
}

// One wave a token: lane l quantises latent channels 8 l .. 8 l + 7 against the
// token's maximum (a wave reduction: the maximum is exact in any order); lanes
// 0-7 also quantise RoPE-key group l.
__global__ __launch_bounds__(256) void append_int8t(uint8_t* pool, int64_t num_pages, const uint16_t* c_kv,
                                                    const uint16_t* k_pe, const int64_t* slots, int n) {
  const int64_t tok = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;   // uniform per wave
  const int lane = threadIdx.x & 63;
  if (tok >= n) return;
  const int64_t slot = slots[tok];
  if (!slot_ok(slot, num_pages)) return;
  uint8_t* page = pool + (slot / kBlock) * kPageInt8Tok;
  const int off = (int)(slot % kBlock);
  const uint16_t* x = c_kv + tok * kDc + 8 * lane;
  float v[8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = bf16_to_f32(x[i]);
    amax = fmaxf(amax, fabsf(v[i]));
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  const float scale = __fdiv_rn(amax, 127.0f);
  int8_t codes[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float q = 0.f;
    if (scale != 0.f) q = fminf(fmaxf(rintf(__fdiv_rn(v[i], scale)), -127.f), 127.f);
    codes[i] = (int8_t)(int)q;
  }
  int8_t* dst = reinterpret_cast<int8_t*>(page + off * 576 + 8 * lane);
#pragma unroll
  for (int i = 0; i < 8; ++i) dst[i] = codes[i];
  if (lane == 0) reinterpret_cast<float*>(page + 64 * 576)[off] = scale;
  if (lane < 8) {
    int8_t rc[8];
    const float s = quant_sym8<8>(k_pe + tok * kDr + lane * 8, rc);
    int8_t* rdst = reinterpret_cast<int8_t*>(page + off * 576 + 512 + lane * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) rdst[i] = rc[i];
    reinterpret_cast<float*>(page + 64 * 576 + 64 * 4)[off * 8 + lane] = s;
  }
}

// FP8 per token: the layout of append_int8t with e4m3 codes and scale = amax / 448.
__global__ __launch_bounds__(256) void append_fp8t(uint8_t* pool, int64_t num_pages, const uint16_t* c_kv,
                                                   const uint16_t* k_pe, const int64_t* slots, int n) {
  const int64_t tok = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;   // uniform per wave
  const int lane = threadIdx.x & 63;
  if (tok >= n) return;
  const int64_t slot = slots[tok];
  if (!slot_ok(slot, num_pages)) return;
  uint8_t* page = pool + (slot / kBlock) * kPageInt8Tok;
  const int off = (int)(slot % kBlock);
  const uint16_t* x = c_kv + tok * kDc + 8 * lane;
  float v[8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = bf16_to_f32(x[i]);
    amax = fmaxf(amax, fabsf(v[i]));
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  const float scale = __fdiv_rn(amax, 448.0f);
  uint8_t* dst = page + off * 576 + 8 * lane;
#pragma unroll
  for (int i = 0; i < 8; ++i) dst[i] = scale != 0.f ? fp8_e4m3_code(__fdiv_rn(v[i], scale)) : (uint8_t)0;
  if (lane == 0) reinterpret_cast<float*>(page + 64 * 576)[off] = scale;
  if (lane < 8) {
    uint8_t rc[8];
    const float s = quant_fp8<8>(k_pe + tok * kDr + lane * 8, rc);
    uint8_t* rdst = page + off * 576 + 512 + lane * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) rdst[i] = rc[i];
    reinterpret_cast<float*>(page + 64 * 576 + 64 * 4)[off * 8 + lane] = s;
  }
}

// ---------------------------------------------------------------------------
// INT8 per channel over 32-token blocks (the report's "per-channel INT8 (32
// blocks)"): the 32 positions 32j..32j+31 of a sequence share, per latent
// channel, scale = max_t |x| / 127; a block is quantised when its 32nd token is
// appended, and until then its rows are kept in bf16.  Page (59,392 B):
//   [64][512] int8 latent codes | [64][64] int8 RoPE-key codes
//   | [2][512] f32 channel scales of blocks 0, 1 | [64][8] f32 RoPE-key scales
//   | [32][512 B] overflow
// An open block b keeps latent channels 0..255 of its row r (bf16, 512 B) in
// code row 32 b + r and channels 256..511 in overflow row r.
// Within one call, the tokens of a block that the call holds must sit at
// consecutive indices in increasing slot order (as a prompt or a decode step
// appends them); a row found neither there nor in the block's open storage
// gives that block unspecified codes, never a fault.
constexpr int kPageInt8c = 59392;
constexpr int kI8cKeyCodes = 64 * 512, kI8cScales = kI8cKeyCodes + 64 * 64, kI8cKeyScales = kI8cScales + 2 * 512 * 4,
              kI8cOverflow = kI8cKeyScales + 64 * 8 * 4;
constexpr int kTBlk = 32;

// Launch 1: one work-group per input token; the group of a token that closes its
// block (position 31 within it) quantises the block, thread t owning latent
// channels 2 t and 2 t + 1 (channels are independent: no reduction across
// threads).  Each of the block's rows comes from the call's input when the call
// holds that position (at index i_close - 31 + rr), else from the block's open
// storage.  The 32 rows are loaded at once (one memory round trip), then each
// channel's maximum and each row's codes are formed from registers; the codes
// overwrite the open storage only after the whole group has read it.
__global__ __launch_bounds__(256) void append_int8c_close(uint8_t* pool, int64_t num_pages, const uint16_t* c_kv,
                                                          const int64_t* slots, int n) {
  const int64_t tok = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t slot = slots[tok];
  if (!slot_ok(slot, num_pages) || slot % kTBlk != kTBlk - 1) return;   // uniform per group
  uint8_t* page = pool + (slot / kBlock) * (int64_t)kPageInt8c;
  const int blk = (int)((slot % kBlock) / kTBlk);
  const int ch = 2 * t;
  // The slots of the call's 31 preceding indices, read unconditionally (index
  // clamped) so that the reads issue together.
  int64_t prev[kTBlk];
#pragma unroll
  for (int rr = 0; rr < kTBlk; ++rr) prev[rr] = slots[max(tok - (kTBlk - 1) + rr, (int64_t)0)];
  uint32_t v[kTBlk];                       // channels ch, ch + 1 of row rr (bf16 pair)
#pragma unroll
  for (int rr = 0; rr < kTBlk; ++rr) {
    const int64_t j = tok - (kTBlk - 1) + rr;  // < n, as tok < n
    const bool in_call = j >= 0 && prev[rr] == slot - (kTBlk - 1) + rr;
    const uint8_t* open = ch < kDc / 2 ? page + (kTBlk * blk + rr) * 512 + 2 * ch
                                       : page + kI8cOverflow + rr * 512 + 2 * (ch - kDc / 2);
    const uint8_t* src = in_call ? reinterpret_cast<const uint8_t*>(c_kv + j * kDc + ch) : open;
    v[rr] = *reinterpret_cast<const uint32_t*>(src);
  }
  float amax0 = 0.f, amax1 = 0.f;
#pragma unroll
  for (int rr = 0; rr < kTBlk; ++rr) {
    amax0 = fmaxf(amax0, fabsf(__uint_as_float(v[rr] << 16)));
    amax1 = fmaxf(amax1, fabsf(__uint_as_float(v[rr] & 0xffff0000u)));
  }
  const float s0 = __fdiv_rn(amax0, 127.0f), s1 = __fdiv_rn(amax1, 127.0f);
  __syncthreads();                         // every row read before any code is written over it
  auto code = [](float x, float sc) {
    float q = 0.f;
    if (sc != 0.f) q = fminf(fmaxf(rintf(__fdiv_rn(x, sc)), -127.f), 127.f);
    return (uint32_t)(int)q & 0xffu;
  };
#pragma unroll
  for (int rr = 0; rr < kTBlk; ++rr) {
    const uint32_t c = code(__uint_as_float(v[rr] << 16), s0) | (code(__uint_as_float(v[rr] & 0xffff0000u), s1) << 8);
    *reinterpret_cast<uint16_t*>(page + (kTBlk * blk + rr) * 512 + ch) = (uint16_t)c;
  }
  float* sc = reinterpret_cast<float*>(page + kI8cScales) + blk * kDc + ch;
  sc[0] = s0;
  sc[1] = s1;
}

// Launch 2 (after launch 1 on the stream): one wave per input token; lanes 0-7
// quantise the RoPE key's 8-groups; the whole wave writes the latent row to its
// block's open storage unless this call also closes the block.
__global__ __launch_bounds__(256) void append_int8c_tok(uint8_t* pool, int64_t num_pages, const uint16_t* c_kv,
                                                        const uint16_t* k_pe, const int64_t* slots, int n) {
  const int64_t tok = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;   // uniform per wave
  const int lane = threadIdx.x & 63;
  if (tok >= n) return;
  const int64_t slot = slots[tok];
  if (!slot_ok(slot, num_pages)) return;
  uint8_t* page = pool + (slot / kBlock) * (int64_t)kPageInt8c;
  const int off = (int)(slot % kBlock), blk = off / kTBlk, rr = off % kTBlk;
  if (lane < 8) {
    int8_t rc[8];
    const float s = quant_sym8<8>(k_pe + tok * kDr + lane * 8, rc);
    int8_t* rdst = reinterpret_cast<int8_t*>(page + kI8cKeyCodes + off * 64 + lane * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) rdst[i] = rc[i];
    reinterpret_cast<float*>(page + kI8cKeyScales)[off * 8 + lane] = s;
  }
  const int64_t jc = tok + (kTBlk - 1 - rr);                 // where this call would hold the block's last row
  const bool closes_here = jc < n && slots[jc] == slot + (kTBlk - 1 - rr);
  if (closes_here) return;
  const u32x4 v = ld16(c_kv + tok * kDc + 8 * lane);
  uint8_t* dst = lane < 32 ? page + (kTBlk * blk + rr) * 512 + 16 * lane : page + kI8cOverflow + rr * 512 + 16 * (lane - 32);
  st16(dst, v);
}

}  // namespace

hipError_t launch_append(int cache_dtype, void* pool, int64_t num_pages, const uint16_t* c_kv,
                         const uint16_t* k_pe, const int64_t* slots, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  uint8_t* p = static_cast<uint8_t*>(pool);
  if (cache_dtype == 0) {
    const int64_t work = (int64_t)n * 72;
    hipLaunchKernelGGL(append_bf16, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, stream, p, num_pages,
                       c_kv, k_pe, slots, n);
  } else if (cache_dtype == 7) {
    const int64_t work = (int64_t)n * 64;                  // one wave a token
    hipLaunchKernelGGL(append_int8c_close, dim3((unsigned)n), dim3(256), 0, stream, p, num_pages, c_kv, slots, n);
    hipLaunchKernelGGL(append_int8c_tok, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, stream, p, num_pages,
                       c_kv, k_pe, slots, n);
  } else if (cache_dtype == 4 || cache_dtype == 5) {
    const int64_t work = (int64_t)n * 64;                  // one wave a token
    hipLaunchKernelGGL(cache_dtype == 4 ? append_int8t : append_fp8t, dim3((unsigned)((work + 255) / 256)),
                       dim3(256), 0, stream, p, num_pages, c_kv, k_pe, slots, n);
  } else {
    const int64_t work = (int64_t)n * 24;
    const dim3 grid((unsigned)((work + 255) / 256));
    if (cache_dtype == 1)
      hipLaunchKernelGGL(append_int8, grid, dim3(256), 0, stream, p, num_pages, c_kv, k_pe, slots, n);
    else if (cache_dtype == 2)
      hipLaunchKernelGGL(append_int4, grid, dim3(256), 0, stream, p, num_pages, c_kv, k_pe, slots, n);
    else if (cache_dtype == 3)
      hipLaunchKernelGGL(append_int4s<false>, grid, dim3(256), 0, stream, p, num_pages, c_kv, k_pe, slots, n);
    else
      hipLaunchKernelGGL(append_int4s<true>, grid, dim3(256), 0, stream, p, num_pages, c_kv, k_pe, slots, n);
  }
  return hipGetLastError();
}

}  // namespace mla
