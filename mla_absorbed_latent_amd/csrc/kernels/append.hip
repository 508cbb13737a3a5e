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
#include "append_row.h"
#include "common.h"
#include "kernels.h"

namespace mla {

namespace {

// One thread per 16-byte chunk of a row (72 a token).
__global__ __launch_bounds__(256) void append_bf16(uint8_t* pool, int64_t num_pages, const uint16_t* c_kv,
                                                   const uint16_t* k_pe, const int64_t* slots, int n) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t tok = gid / 72;
  const int chunk = (int)(gid % 72);
  if (tok >= n) return;
  const int64_t slot = slots[tok];
  if (!slot_ok(slot, num_pages)) return;
  row_bf16(pool, slot, c_kv + tok * kDc, k_pe + tok * kDr, chunk);
}

// One thread per quantisation group: 24 a token (16 latent groups of 32, then 8
// RoPE-key groups of 8), for INT8 and the three INT4 layouts.
#define MLA_APPEND_GROUPS(NAME, CALL)                                                                          \
  __global__ __launch_bounds__(256) void NAME(uint8_t* pool, int64_t num_pages, const uint16_t* c_kv,            \
                                              const uint16_t* k_pe, const int64_t* slots, int n) {                \
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;                                                 \
    const int64_t tok = gid / 24;                                                                                \
    const int grp = (int)(gid % 24);                                                                             \
    if (tok >= n) return;                                                                                        \
    const int64_t slot = slots[tok];                                                                             \
    if (!slot_ok(slot, num_pages)) return;                                                                       \
    CALL(pool, slot, c_kv + tok * kDc, k_pe + tok * kDr, grp);                                                   \
  }
MLA_APPEND_GROUPS(append_int8, row_int8)
MLA_APPEND_GROUPS(append_int4, row_int4)
MLA_APPEND_GROUPS(append_int4s, row_int4s<false>)
MLA_APPEND_GROUPS(append_int4s_k4, row_int4s<true>)
#undef MLA_APPEND_GROUPS

// One wave a token: per-token INT8 (append_int8t) or e4m3 (append_fp8t).
#define MLA_APPEND_TOK(NAME, FP8)                                                                              \
  __global__ __launch_bounds__(256) void NAME(uint8_t* pool, int64_t num_pages, const uint16_t* c_kv,            \
                                              const uint16_t* k_pe, const int64_t* slots, int n) {                \
    const int64_t tok = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6; /* uniform per wave */                   \
    if (tok >= n) return;                                                                                        \
    const int64_t slot = slots[tok];                                                                             \
    if (!slot_ok(slot, num_pages)) return;                                                                       \
    row_tok<FP8>(pool, slot, c_kv + tok * kDc, k_pe + tok * kDr, threadIdx.x & 63);                              \
  }
MLA_APPEND_TOK(append_int8t, false)
MLA_APPEND_TOK(append_fp8t, true)
#undef MLA_APPEND_TOK

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

// Launch 2 (after launch 1 on the stream): one wave per input token, the per-token
// part (RoPE key; the latent row to the open storage unless this call closes its block).
__global__ __launch_bounds__(256) void append_int8c_tok(uint8_t* pool, int64_t num_pages, const uint16_t* c_kv,
                                                        const uint16_t* k_pe, const int64_t* slots, int n) {
  const int64_t tok = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;   // uniform per wave
  if (tok >= n) return;
  const int64_t slot = slots[tok];
  if (!slot_ok(slot, num_pages)) return;
  row_int8c_tok(pool, slot, c_kv + tok * kDc, k_pe + tok * kDr, threadIdx.x & 63, int8c_closes_here(slots, n, tok, slot));
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
      hipLaunchKernelGGL(append_int4s, grid, dim3(256), 0, stream, p, num_pages, c_kv, k_pe, slots, n);
    else
      hipLaunchKernelGGL(append_int4s_k4, grid, dim3(256), 0, stream, p, num_pages, c_kv, k_pe, slots, n);
  }
  return hipGetLastError();
}

}  // namespace mla
