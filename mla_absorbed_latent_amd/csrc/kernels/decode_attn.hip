// decode_attn.hip -- split-KV absorbed MLA decode attention for gfx950.
//
// What is computed ("DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界" §2.2-§2.4 and
// §6.1; "手搓 MLA:从 MHA 到 weight absorption" §四): every query head of a sequence
// attends to the same cached rows [c_t (512) ; k_pe_t (64)], i.e. MQA with one
// shared "KV head" of width 576 for scores and 512 for values.  Per work item
// (a run of a sequence's pages) and head:
//   s_t = scale * q_abs . row_t,  o = sum_t e^{s_t-m} c_t / l,  lse = m + ln l.
// Quantised caches ("DeepSeek-V2-Lite MLA 吸收式 KV 缓存优化 — 完整实验报告" §3.2/§4.1)
// are dequantised once per tile into the same fp16 tile layout.
//
// gfx950 design
//   * One work-group (4 wave64s) per work item; the item's tokens stream through
//     LDS in tiles of fp16 rows (1,152 B, 16-byte chunks XOR-swizzled by row so
//     that every MFMA operand fetch is free of bank conflicts).
//   * Tiles are staged through VGPRs: each thread loads its share of the next
//     tile one tile ahead, widens bf16 -> fp16 (or dequantises) in registers and
//     writes it to the other LDS buffer.  Loads and conversions are woven into
//     the matrix-instruction stream, so they run in the MFMA shadow.
//   * H = 128 (per 32-token tile): wave w computes the scores of heads
//     32w..32w+31 (S^T = K . Q^T, 36 x mfma 32x32x16, K from LDS, Q^T mostly in
//     VGPRs), writes fp16 P to a small LDS exchange buffer, and then the value
//     product for features 128w..128w+127 of all 128 heads (O^T += V^T . P^T,
//     32 x mfma 32x32x16, V^T read transposed with ds_read_b64_tr_b16).  Every
//     wave thus reads all of K but only a quarter of V: on this part the LDS,
//     more than the matrix cores, bounds the rate, and the chip's power limit
//     bounds the clock.
//   * H = 16: each wave takes 16 tokens of a 64-token page for all 16 heads
//     (mfma 16x16x32 scores, 16x16x16 values); the four waves' (max, sum, O) are
//     merged through LDS at the end.
//   * Softmax in the log2 domain.  H = 128 fixes each head's reference max at its
//     first non-empty tile and never rescales O inside the loop (P <= 2^15 fits
//     fp16); if a later tile exceeds that by more than 2^15 the item is redone
//     against exact maxima (one scores-only pass, one accumulate pass).  H = 16
//     rescales lazily (only when the max grows by more than 2^8).
//   * Tokens past the item's end, or on pages whose id is outside the pool, are
//     loaded from an all-zero page and masked to -inf.
#include <type_traits>

#include "common.h"
#include "decode_attn.h"
#include "item_range.h"

namespace mla {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;         // lazy-rescale threshold (log2 units), H = 16
constexpr float kTauFixed = 15.0f;   // fixed-reference headroom (log2 units), H = 128: P <= 2^15

constexpr int kRowLds = kDk * 2;                    // 1,152 B: one fp16 token row in LDS

// LDS tile layout: fp16 rows of 1,152 B (72 chunks of 16 B).  The 16-byte chunk
// index is XORed (within its aligned group of 8) with a function of row bits 1..3,
// chosen per kernel so that the MFMA operand fetches of that kernel are free of
// bank conflicts on the 64-bank LDS: the row stride is 32 banks, so rows r and
// r ^ 1 never collide and the XOR only has to separate rows that share parity.
//   kSwz128: for 16 consecutive rows reading one chunk (score operand) and for
//            4 rows x 32 B transposed reads (value operand).
//   kSwz16:  the same two patterns at the 16-head shapes.
constexpr int kSwz128 = 0, kSwz16 = 1;
template <int kSwz>
__device__ __forceinline__ int swz_key(int row) {
  const int m = (row >> 1) & 7;
  return kSwz == kSwz128 ? (((m & 1) << 2) | (m >> 1)) : (((m & 3) << 1) | (m >> 2));
}
template <int kSwz>
__device__ __forceinline__ uint32_t swz(int row, int chunk) {
  return (uint32_t)(row * kRowLds + 16 * (chunk ^ swz_key<kSwz>(row)));
}

struct ItemRange {
  int b, t_begin, t_end, out_row;
  bool ok;
};

__device__ __forceinline__ ItemRange item_range(const DecodeArgs& a) {
  ItemRange r;
  const mla_work_item it = a.items[blockIdx.x];
  r.b = it.seq;
  r.out_row = it.out_row;
  r.ok = it.seq >= 0 && it.seq < a.batch && it.out_row >= 0 && it.out_row < a.n_items && it.first_page >= 0 &&
         it.n_pages >= 0;
  if (!r.ok) { r.t_begin = r.t_end = 0; return r; }
  const TokenRange tr = item_token_range(it.first_page, it.n_pages, a.max_pages, a.seq_lens[it.seq], kBlock);
  r.t_begin = tr.t_begin;
  r.t_end = tr.t_end;
  return r;
}

// Physical page of logical token t of sequence b, or -1 when out of range.
__device__ __forceinline__ int64_t page_of(const DecodeArgs& a, int b, int t) {
  const int lp = t / kBlock;
  if (lp < 0 || lp >= a.max_pages) return -1;
  const int64_t p = a.block_table[(int64_t)b * a.max_pages + lp];
  return (p >= 0 && p < a.num_pages) ? p : -1;
}

// Every pipeline looks its pages up in an LDS copy of the item's block-table
// slice, refreshed every kSegPages pages: a global read of the table inside a
// tile loop would make the compiler's wait for it also drain the tile prefetch
// issued before it (vector-memory counters retire in order).
constexpr int kSegPages = 1024;

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] = 7 |
// lgkmcnt[11:8] = 15 | vmcnt[5:4] in bits [15:14]).
template <int kN>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((kN & 15) | (7 << 4) | (15 << 8) | ((kN >> 4) << 14));
}
__device__ __forceinline__ void fill_ptab(const DecodeArgs& a, int b, int t0, int t1, int32_t* ptab) {
  const int n = (t1 - t0 + kBlock - 1) / kBlock;
  for (int i = threadIdx.x; i < n; i += blockDim.x) ptab[i] = (int32_t)page_of(a, b, t0 + i * kBlock);
}

// ===========================================================================
// Register-prefetch tile loaders: issue() loads a tile of physical page `page`
// (-1: out of range) into registers, commit() writes it as fp16 rows into an LDS
// buffer.  kTok tokens (32 or 64), starting at a multiple of kTok within a page.
// Thread tid owns token (tid >> 3) of each 32-token pass and the 16-byte output
// chunks (tid & 7) + 8k, k = 0..8 (k = 8 is the RoPE key), so all offsets are
// affine in k.  Both are free of branches, so that a caller can interleave them
// with matrix instructions: a row past t_end, or on a page out of range, is
// loaded from an all-zero page and so written as zeros.
// ===========================================================================

// Rows that are out of range are read from this all-zero page instead (device
// globals start zeroed; it is as large as the largest page format, so every
// field offset stays valid), and every cache format decodes zero bytes to zeros.
__device__ __attribute__((aligned(256))) uint8_t g_zero_page[kBlock * kRowBytesBf16];

// Loader thread index: a loader spreads a tile over 256 threads, work-group
// threads kTid0 .. kTid0 + 255 (the whole 128-head work-group, or the staging
// waves of the 16-head one).
template <int kTid0>
__device__ __forceinline__ int ltid() { return (int)threadIdx.x - kTid0; }

// Base of page `page`, or of the zero page when the row is out of range.  Both
// operands are selected, so that no branch (and no exec-masked region) forms
// around the multiply inside a tile loop.
__device__ __forceinline__ const uint8_t* page_base(const DecodeArgs& a, int64_t page, bool ok, int64_t page_bytes) {
  const uint8_t* base = ok ? a.pool : g_zero_page;
  return base + (ok ? page : 0) * page_bytes;
}


template <int kTok, int kSwz, int kTid0 = 0>
struct LoaderBf16Reg {
  static constexpr int kPass = kTok / 32;
  static constexpr int kScorePrefetch = 3;   // K fragments in flight in the 128-head score loop
  u32x4 r[9 * kPass];

  __device__ __forceinline__ bool issue(const DecodeArgs& a, int64_t page, int t0, int t_end) {
    const int tok = ltid<kTid0>() >> 3;
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const bool ok = page >= 0 && t0 + 32 * p + tok < t_end;
      const uint8_t* src = page_base(a, page, ok, kBlock * kRowBytesBf16) +
                           ((t0 % kBlock) + 32 * p + tok) * kRowBytesBf16 + 16 * (ltid<kTid0>() & 7);
#pragma unroll
      for (int k = 0; k < 9; ++k) r[9 * p + k] = ld16_stream(src + 128 * k);
    }
    return page >= 0;
  }
  // Stepwise issue (one pass, 128-head pipeline): begin() sets this lane's row
  // source; load_step<I> (after store_step<I>) reloads chunk I / 2 once its
  // store is done (odd I), so the loads trickle out one per two MFMAs and have a
  // whole tile step to arrive before they are widened.
  const uint8_t* src;
  __device__ __forceinline__ void begin(const DecodeArgs& a, int64_t page, int t0, int t_end) {
    const int tok = ltid<kTid0>() >> 3;
    const bool ok = page >= 0 && t0 + tok < t_end;
    src = page_base(a, page, ok, kBlock * kRowBytesBf16) + ((t0 % kBlock) + tok) * kRowBytesBf16 + 16 * (ltid<kTid0>() & 7);
  }
  template <int I>
  __device__ __forceinline__ void load_step() {
    if constexpr (I % 2 == 1) r[I / 2] = ld16_stream(src + 128 * (I / 2));
  }
  // Stepwise commit: step 2c widens the first half of chunk c in place, step
  // 2c+1 the second half, and stores the chunk.
  static constexpr int kStoreSteps = 18;
  template <int I>
  __device__ __forceinline__ void store_step(char* lds_buf) {
    constexpr int kc = I / 2, d0 = 2 * (I % 2);
#pragma unroll
    for (int d = d0; d < d0 + 2; ++d) {
      uint32_t v = bf16x2_to_f16x2(r[kc][d]);
      asm volatile("" : "+v"(v));   // keep the conversion in this step, not sunk to the store
      r[kc][d] = v;
    }
    if constexpr (I % 2 == 1)
      *reinterpret_cast<u32x4*>(lds_buf + swz<kSwz>(ltid<kTid0>() >> 3, ltid<kTid0>() & 7) + 128 * kc) = r[kc];
  }
  __device__ __forceinline__ void commit(char* lds_buf) {
    const int tok = ltid<kTid0>() >> 3;
    char* dst = lds_buf + swz<kSwz>(tok, ltid<kTid0>() & 7);
#pragma unroll
    for (int p = 0; p < kPass; ++p)
#pragma unroll
      for (int k = 0; k < 9; ++k)
        *reinterpret_cast<u32x4*>(dst + 32 * p * kRowLds + 128 * k) = bf16x8_to_f16x8(r[9 * p + k]);
  }
};

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Four int8 codes -> four fp16 values code * s (s already fp16).  0x6400 | (code ^ 0x80)
// is the fp16 number 1024 + code + 128, exactly; subtracting 1152 leaves the code.
__device__ __forceinline__ u32x2 int8x4_to_f16(uint32_t c, half2v s) {
  const uint32_t u = c ^ 0x80808080u;
  const uint32_t h0 = 0x64006400u | (u & 0xffu) | ((u & 0xff00u) << 8);
  const uint32_t h1 = 0x64006400u | ((u >> 16) & 0xffu) | ((u >> 8) & 0xff0000u);
  const half2v bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  return u32x2{__builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2v, h0) + bias) * s),
               __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2v, h1) + bias) * s)};
}
// The same values, each fp16 pair assembled by one byte permute (bytes 0-3 of
// the permute's 8-byte source are u, bytes 4-7 the constant 0x64 bytes).  The two
// selectors occupy VGPRs, so only the staging waves of the 16-head kernel,
// which have registers to spare, use this form.
__device__ __forceinline__ u32x2 int8x4_to_f16_perm(uint32_t c, half2v s) {
  const uint32_t u = c ^ 0x80808080u;
  const uint32_t h0 = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);   // (u.b0, u.b1)
  const uint32_t h1 = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);   // (u.b2, u.b3)
  const half2v bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  return u32x2{__builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2v, h0) + bias) * s),
               __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2v, h1) + bias) * s)};
}

// Four e4m3 codes -> four fp16 values value(code) * s256 / 256.  Placing byte b in
// bits 8-15 of a 16-bit lane and shifting its low seven bits down by one gives
// (b & 0x7f) << 7 | (b & 0x80) << 8: sign, exponent and mantissa fields line up
// with fp16's, and with the exponent biases 7 and 15 that bit pattern is the fp16
// number value(b) * 2^-8, exactly, subnormals included.  s256 is the scale times
// 256.
__device__ __forceinline__ uint32_t fp8x2_f16_bits(uint32_t t) {
  return ((t >> 1) & 0x3f803f80u) | (t & 0x80008000u);
}
__device__ __forceinline__ u32x2 fp8x4_to_f16(uint32_t c, half2v s256) {
  const uint32_t t0 = __builtin_amdgcn_perm(0u, c, 0x010c000cu);   // (0, b0, 0, b1)
  const uint32_t t1 = __builtin_amdgcn_perm(0u, c, 0x030c020cu);   // (0, b2, 0, b3)
  return u32x2{__builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, fp8x2_f16_bits(t0)) * s256),
               __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, fp8x2_f16_bits(t1)) * s256)};
}
// Codes of the byte-coded formats -> fp16 (kFp8: e4m3, else int8), and the fp16
// factor their scale s becomes.
template <bool kFp8>
__device__ __forceinline__ u32x2 codes4_to_f16(uint32_t c, half2v s) {
  if constexpr (kFp8) return fp8x4_to_f16(c, s);
  else return int8x4_to_f16(c, s);
}
template <bool kFp8>
__device__ __forceinline__ u32x2 codes4_to_f16_perm(uint32_t c, half2v s) {
  if constexpr (kFp8) return fp8x4_to_f16(c, s);
  else return int8x4_to_f16_perm(c, s);
}
template <bool kFp8>
__device__ __forceinline__ _Float16 code_scale_h(float s) {
  return (_Float16)(kFp8 ? s * 256.f : s);
}

// INT8 page: [64][576] codes | [64][16] f32 latent scales | [64][8] f32 key scales.
// Per-token INT8 (kTok1): [64][576] codes | [64] f32 latent scales | [64][8] f32
// key scales; every latent chunk of a token takes the token's one scale.
// FP8 per token (kFp8, with kTok1): the same page with e4m3 codes.
template <int kTok, int kSwz, int kTid0 = 0, bool kTok1 = false, bool kFp8 = false>
struct LoaderInt8Reg {
  static constexpr int kPass = kTok / 32;
  static constexpr int kScorePrefetch = 3;
  static constexpr int kPage = kBlock * (kTok1 ? 612 : 672);
  static constexpr int kKeyScales = 64 * 576 + (kTok1 ? 64 * 4 : 64 * 64);   // byte offset of the key scales
  u32x2 c[9 * kPass];
  float s[9 * kPass];
  // Float index of latent chunk k's scale for (row, c8).
  static __device__ __forceinline__ int scale_index(int row, int c8, int k) {
    return kTok1 ? row : row * 16 + (c8 >> 2) + 2 * k;
  }

  __device__ __forceinline__ bool issue(const DecodeArgs& a, int64_t page, int t0, int t_end) {
    const int tok = ltid<kTid0>() >> 3, c8 = ltid<kTid0>() & 7;
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const bool ok = page >= 0 && t0 + 32 * p + tok < t_end;
      const int row = (t0 % kBlock) + 32 * p + tok;
      const uint8_t* pg = page_base(a, page, ok, kPage);
      const uint8_t* codes = pg + row * 576 + 8 * c8;
      const float* cs = reinterpret_cast<const float*>(pg + 64 * 576);
      const float* ks = reinterpret_cast<const float*>(pg + kKeyScales) + row * 8 + c8;
#pragma unroll
      for (int k = 0; k < 9; ++k) {
        c[9 * p + k] = *reinterpret_cast<const u32x2*>(codes + 64 * k);
        s[9 * p + k] = k < 8 ? cs[scale_index(row, c8, k)] : ks[0];
      }
    }
    return page >= 0;
  }
  // Stepwise issue (one pass, 128-head pipeline): begin() sets this lane's page
  // and row; load_step<I> (after store_step<I>) reloads chunk I / 2 once its
  // store is done (odd I).
  const uint8_t* pg;
  int row;
  __device__ __forceinline__ void begin(const DecodeArgs& a, int64_t page, int t0, int t_end) {
    const int tok = ltid<kTid0>() >> 3;
    const bool ok = page >= 0 && t0 + tok < t_end;
    pg = page_base(a, page, ok, kPage);
    row = (t0 % kBlock) + tok;
  }
  template <int I>
  __device__ __forceinline__ void load_step() {
    if constexpr (I % 2 == 1) {
      constexpr int k = I / 2;
      const int c8 = ltid<kTid0>() & 7;
      c[k] = *reinterpret_cast<const u32x2*>(pg + row * 576 + 8 * c8 + 64 * k);
      if constexpr (k < 8) s[k] = reinterpret_cast<const float*>(pg + 64 * 576)[scale_index(row, c8, k)];
      else s[k] = reinterpret_cast<const float*>(pg + kKeyScales)[row * 8 + c8];
    }
  }
  // Stepwise commit: step 2c dequantises the first four codes of chunk c, step
  // 2c+1 the other four and stores the chunk.
  static constexpr int kStoreSteps = 18 * kPass;
  u32x2 part;
  template <int I>
  __device__ __forceinline__ void store_step(char* lds_buf) {
    constexpr int kc = I / 2, p = kc / 9, k = kc % 9;
    const _Float16 sh = code_scale_h<kFp8>(s[kc]);
    const half2v s2 = {sh, sh};
    if constexpr (I % 2 == 0) {
      part = codes4_to_f16<kFp8>(c[kc][0], s2);
    } else {
      const u32x2 hi = codes4_to_f16<kFp8>(c[kc][1], s2);
      *reinterpret_cast<u32x4*>(lds_buf + swz<kSwz>(ltid<kTid0>() >> 3, ltid<kTid0>() & 7) + 32 * p * kRowLds + 128 * k) =
          u32x4{part[0], part[1], hi[0], hi[1]};
    }
  }
  __device__ __forceinline__ void commit(char* lds_buf) {
    const int tok = ltid<kTid0>() >> 3;
    char* dst = lds_buf + swz<kSwz>(tok, ltid<kTid0>() & 7);
#pragma unroll
    for (int p = 0; p < kPass; ++p)
#pragma unroll
      for (int k = 0; k < 9; ++k) {
        const _Float16 sh = code_scale_h<kFp8>(s[9 * p + k]);
        const half2v s2 = {sh, sh};
        const u32x2 lo = codes4_to_f16<kFp8>(c[9 * p + k][0], s2), hi = codes4_to_f16<kFp8>(c[9 * p + k][1], s2);
        *reinterpret_cast<u32x4*>(dst + 32 * p * kRowLds + 128 * k) = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
  }
};

// INT8 per channel over 32-token blocks: page [64][512] latent codes | [64][64]
// key codes | [2][512] f32 channel scales (one row per block) | [64][8] f32 key
// scales | [32][256] bf16 overflow.  A block is closed once its 32nd token is
// written (codes and channel scales); the one open block of a sequence keeps its
// rows in bf16, channels 0..255 in the row's own code row and 256..511 in
// overflow row (row % 32).  The RoPE key is INT8 per 8-group in every row.
constexpr int kPageInt8c = 59392;
constexpr int kI8cKeyCodes = 64 * 512, kI8cScales = kI8cKeyCodes + 64 * 64, kI8cKeyScales = kI8cScales + 2 * 512 * 4,
              kI8cOverflow = kI8cKeyScales + 64 * 8 * 4;
static_assert(kI8cOverflow + 32 * 512 == kPageInt8c, "page layout");

// Byte offset of 16-byte LDS chunk q (0..71) of tile row `row`.
template <int kSwz>
__device__ __forceinline__ uint32_t swz_chunk(int row, int q) { return swz<kSwz>(row, q & 7) + 128 * (q >> 3); }

// Closed blocks, 32-token tiles (a tile is one block: tiles start at multiples
// of 32 and a closed range ends at one).  Threads are laid out down the
// channels, so that each needs 8 of the block's channel scales: thread t owns
// the 8-channel chunk q = t % 64 of tile rows 8 (t / 64) + m, m = 0..7; and the
// 8 key codes of group t % 8 of row t / 8.  A whole tile is in range or not.
template <int kSwz>
struct LoaderInt8cReg {
  static constexpr int kScorePrefetch = 3;
  u32x2 c[8];                 // codes of chunk q, rows 8 w + m
  floatx4 sv[2];              // f32 scales of channels 8 q .. 8 q + 7
  uint32_t h2[4];             // the same as fp16 pairs, formed at the first store step
  u32x2 kc;                   // key codes of group t % 8 of row t / 8
  float ks;
  const uint8_t* pg;          // the tile's page (uniform: the whole tile is in range or not)
  uint32_t row0;              // first tile row within the page (0 or 32)

  __device__ __forceinline__ void begin(const DecodeArgs& a, int64_t page, int t0, int t_end) {
    pg = page_base(a, page, page >= 0 && t0 < t_end, kPageInt8c);
    row0 = (uint32_t)(t0 % kBlock);
  }
  __device__ __forceinline__ void load_codes(int m) {
    const uint32_t t = threadIdx.x;
    const uint32_t off = (row0 + 8 * (t >> 6)) * 512 + 8 * (t & 63);
    c[m] = *reinterpret_cast<const u32x2*>(pg + off + 512 * m);
  }
  __device__ __forceinline__ void load_scales() {
    const uint32_t off = kI8cScales + (row0 >> 5) * 2048 + 32 * (threadIdx.x & 63);
    sv[0] = *reinterpret_cast<const floatx4*>(pg + off);
    sv[1] = *reinterpret_cast<const floatx4*>(pg + off + 16);
  }
  __device__ __forceinline__ void load_key() {
    const uint32_t row = row0 + (threadIdx.x >> 3), g8 = threadIdx.x & 7;
    kc = *reinterpret_cast<const u32x2*>(pg + (kI8cKeyCodes + row * 64 + 8 * g8));
    ks = *reinterpret_cast<const float*>(pg + (kI8cKeyScales + row * 32 + 4 * g8));
  }
  __device__ __forceinline__ bool issue(const DecodeArgs& a, int64_t page, int t0, int t_end) {
    begin(a, page, t0, t_end);
#pragma unroll
    for (int m = 0; m < 8; ++m) load_codes(m);
    load_scales();
    load_key();
    return page >= 0;
  }
  __device__ __forceinline__ void make_h2() {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      h2[j] = __builtin_bit_cast(uint32_t, half2v{(_Float16)sv[j >> 1][2 * (j & 1)], (_Float16)sv[j >> 1][2 * (j & 1) + 1]});
  }
  // Four codes (channels 4 d .. 4 d + 3 of the chunk) -> two fp16 pairs.
  __device__ __forceinline__ u32x2 deq4(uint32_t w, int d) const {
    const uint32_t u = w ^ 0x80808080u;
    const half2v bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const uint32_t lo = 0x64006400u | (u & 0xffu) | ((u & 0xff00u) << 8);
    const uint32_t hi = 0x64006400u | ((u >> 16) & 0xffu) | ((u >> 8) & 0xff0000u);
    return u32x2{__builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2v, lo) + bias) * __builtin_bit_cast(half2v, h2[2 * d])),
                 __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2v, hi) + bias) * __builtin_bit_cast(half2v, h2[2 * d + 1]))};
  }
  __device__ __forceinline__ void store_key(char* lds_buf) const {
    const _Float16 k = (_Float16)ks;
    const u32x2 lo = int8x4_to_f16(kc[0], half2v{k, k}), hi = int8x4_to_f16(kc[1], half2v{k, k});
    *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(threadIdx.x >> 3, 64 + (threadIdx.x & 7))) =
        u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
  // Stepwise commit (steps 2 m, 2 m + 1: row m's chunk; 16, 17: the key) and
  // reload, as for the other formats.  The scales are turned into fp16 pairs at
  // step 0 and reloaded at step 1.
  static constexpr int kStoreSteps = 18;
  u32x2 part;
  template <int I>
  __device__ __forceinline__ void store_step(char* lds_buf) {
    constexpr int m = I / 2;
    if constexpr (m < 8) {
      if constexpr (I == 0) make_h2();
      if constexpr (I % 2 == 0) {
        part = deq4(c[m][0], 0);
      } else {
        const u32x2 hi = deq4(c[m][1], 1);
        *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(8 * (threadIdx.x >> 6) + m, threadIdx.x & 63)) =
            u32x4{part[0], part[1], hi[0], hi[1]};
      }
    } else if constexpr (I % 2 == 1) {
      store_key(lds_buf);
    }
  }
  template <int I>
  __device__ __forceinline__ void load_step() {
    if constexpr (I % 2 == 1) {
      constexpr int m = I / 2;
      if constexpr (m < 8) load_codes(m);
      else load_key();
      if constexpr (I == 1) load_scales();
    }
  }
  __device__ __forceinline__ void commit(char* lds_buf) {
    make_h2();
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const u32x2 lo = deq4(c[m][0], 0), hi = deq4(c[m][1], 1);
      *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(8 * (threadIdx.x >> 6) + m, threadIdx.x & 63)) =
          u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    store_key(lds_buf);
  }
};

// The open block, 32-token tiles: rows in bf16 as in LoaderBf16Reg (thread t:
// row t / 8, latent chunks t % 8 + 8 k), chunks 0..31 from the code row and
// 32..63 from the overflow row; the key as in LoaderInt8cReg.  Rows past t_end
// read the zero page.
template <int kSwz>
struct LoaderInt8cOpenReg {
  static constexpr int kScorePrefetch = 3;
  u32x4 r[8];
  u32x2 kc;
  float ks;
  const uint8_t* pg;
  int row;

  __device__ __forceinline__ void begin(const DecodeArgs& a, int64_t page, int t0, int t_end) {
    const int tok = threadIdx.x >> 3;
    pg = page_base(a, page, page >= 0 && t0 + tok < t_end, kPageInt8c);
    row = t0 % kBlock + tok;
  }
  template <int K>
  __device__ __forceinline__ void load_chunk() {
    const int q = (threadIdx.x & 7) + 8 * K;
    if constexpr (K < 4) r[K] = ld16_stream(pg + row * 512 + 16 * q);
    else r[K] = ld16_stream(pg + kI8cOverflow + (row % 32) * 512 + 16 * (q - 32));
  }
  __device__ __forceinline__ void load_key() {
    const int g8 = threadIdx.x & 7;
    kc = *reinterpret_cast<const u32x2*>(pg + kI8cKeyCodes + row * 64 + 8 * g8);
    ks = reinterpret_cast<const float*>(pg + kI8cKeyScales)[row * 8 + g8];
  }
  __device__ __forceinline__ bool issue(const DecodeArgs& a, int64_t page, int t0, int t_end) {
    begin(a, page, t0, t_end);
    load_chunk<0>();
    load_chunk<1>();
    load_chunk<2>();
    load_chunk<3>();
    load_chunk<4>();
    load_chunk<5>();
    load_chunk<6>();
    load_chunk<7>();
    load_key();
    return page >= 0;
  }
  __device__ __forceinline__ void store_key(char* lds_buf) const {
    const _Float16 k = (_Float16)ks;
    const u32x2 lo = int8x4_to_f16(kc[0], half2v{k, k}), hi = int8x4_to_f16(kc[1], half2v{k, k});
    *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(threadIdx.x >> 3, 64 + (threadIdx.x & 7))) =
        u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
  static constexpr int kStoreSteps = 18;
  template <int I>
  __device__ __forceinline__ void store_step(char* lds_buf) {
    constexpr int k = I / 2;
    if constexpr (I % 2 == 1) {
      if constexpr (k < 8)
        *reinterpret_cast<u32x4*>(lds_buf + swz<kSwz>(threadIdx.x >> 3, threadIdx.x & 7) + 128 * k) = bf16x8_to_f16x8(r[k]);
      else
        store_key(lds_buf);
    }
  }
  template <int I>
  __device__ __forceinline__ void load_step() {
    if constexpr (I % 2 == 1) {
      if constexpr (I / 2 < 8) load_chunk<I / 2>();
      else load_key();
    }
  }
  __device__ __forceinline__ void commit(char* lds_buf) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      *reinterpret_cast<u32x4*>(lds_buf + swz<kSwz>(threadIdx.x >> 3, threadIdx.x & 7) + 128 * k) = bf16x8_to_f16x8(r[k]);
    store_key(lds_buf);
  }
};

// INT4 page: [64][256] latent nibbles | [64][64] int8 key codes | [64][16] f32 scales
//            | [64][16] f32 zeros | [64][8] f32 key scales.
// Symmetric INT4 (kSym) drops the zeros: a nibble holds q + 8 and decodes to
// (nibble - 8) * scale.
// kKey4 (with kSym): the RoPE key as symmetric INT4 too, 8 nibbles per lane
// ([64][32] key nibbles in place of the [64][64] codes; 384 B/token).
template <int kTok, int kSwz, int kTid0 = 0, bool kSym = false, bool kKey4 = false>
struct LoaderInt4Reg {
  static constexpr int kPass = kTok / 32;
  static constexpr int kScorePrefetch = 2;    // its staging registers leave room for two
  static constexpr int kPage = kBlock * (kKey4 ? 384 : (kSym ? 416 : 480));
  static constexpr int kMeta = 64 * 256 + 64 * (kKey4 ? 32 : 64);   // byte offset of the scales
  static constexpr int kKeyScales = kSym ? 64 * 16 : 2 * 64 * 16;   // float offset of the key scales after the scales
  uint32_t n[8 * kPass];     // 8 nibbles (latent chunk k) per dword
  u32x2 kc[kPass];           // 8 key codes (chunk 8); kKey4: 8 key nibbles in kc[p][0]
  float s[9 * kPass];        // scale per chunk (k = 8: key scale)
  float z[kSym ? 1 : 8 * kPass];   // zero point per latent chunk (asymmetric only)

  __device__ __forceinline__ bool issue(const DecodeArgs& a, int64_t page, int t0, int t_end) {
    const int tok = ltid<kTid0>() >> 3, c8 = ltid<kTid0>() & 7;
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const bool ok = page >= 0 && t0 + 32 * p + tok < t_end;
      const int row = (t0 % kBlock) + 32 * p + tok;
      const uint8_t* pg = page_base(a, page, ok, kPage);
      const float* scales = reinterpret_cast<const float*>(pg + kMeta) + row * 16 + (c8 >> 2);
      const float* zeros = scales + 64 * 16;
      const float* kscales = reinterpret_cast<const float*>(pg + kMeta) + kKeyScales + row * 8 + c8;
      const uint8_t* nib = pg + row * 256 + 4 * c8;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        n[8 * p + k] = *reinterpret_cast<const uint32_t*>(nib + 32 * k);
        s[9 * p + k] = scales[2 * k];
        if constexpr (!kSym) z[8 * p + k] = zeros[2 * k];
      }
      if constexpr (kKey4) kc[p][0] = *reinterpret_cast<const uint32_t*>(pg + 64 * 256 + row * 32 + 4 * c8);
      else kc[p] = *reinterpret_cast<const u32x2*>(pg + 64 * 256 + row * 64 + 8 * c8);
      s[9 * p + 8] = kscales[0];
    }
    return page >= 0;
  }
  // Byte j of nibble word w (elements 2j, 2j+1) -> two fp16 values (q - 8) * s + z8,
  // z8 = z + 8 s (symmetric: (q - 8) * s).  Centring the code keeps the fp16
  // zero point near the group's midpoint, small for centred data, so its
  // rounding (and the scale's) moves a value by far less than with z itself.
  static __device__ __forceinline__ uint32_t nib2(uint32_t w, int j, half2v s2, half2v z2) {
    constexpr float kBias = -1032.0f;
    const half2v bias = {(_Float16)kBias, (_Float16)kBias};
    const uint32_t byte = (w >> (8 * j)) & 0xffu;
    // (element 2j, element 2j+1) = (low nibble, high nibble) as fp16 1024 + q
    const uint32_t h = 0x64006400u | (byte & 0xfu) | ((byte >> 4) << 16);
    const half2v qv = __builtin_bit_cast(half2v, h) + bias;
    if constexpr (kSym) return __builtin_bit_cast(uint32_t, qv * s2);
    else return __builtin_bit_cast(uint32_t, qv * s2 + z2);
  }
  // fp16 zero point of latent chunk i (scale s): z + 8 s, formed in fp32.
  __device__ __forceinline__ _Float16 zero_h(int i, float s) const {
    if constexpr (kSym) return (_Float16)0.0f;
    else return (_Float16)fmaf(8.0f, s, z[i]);
  }
  // Stepwise issue (one pass, 128-head pipeline): begin() sets this lane's page
  // and row; load_step<I> (after store_step<I>) reloads chunk I / 2 once its
  // store is done (odd I).
  const uint8_t* pg;
  int row;
  __device__ __forceinline__ void begin(const DecodeArgs& a, int64_t page, int t0, int t_end) {
    const int tok = ltid<kTid0>() >> 3;
    const bool ok = page >= 0 && t0 + tok < t_end;
    pg = page_base(a, page, ok, kPage);
    row = (t0 % kBlock) + tok;
  }
  template <int I>
  __device__ __forceinline__ void load_step() {
    if constexpr (I % 2 == 1) {
      constexpr int k = I / 2;
      const int c8 = ltid<kTid0>() & 7;
      const float* meta = reinterpret_cast<const float*>(pg + kMeta);
      if constexpr (k < 8) {
        n[k] = *reinterpret_cast<const uint32_t*>(pg + row * 256 + 4 * c8 + 32 * k);
        s[k] = meta[row * 16 + (c8 >> 2) + 2 * k];
        if constexpr (!kSym) z[k] = meta[64 * 16 + row * 16 + (c8 >> 2) + 2 * k];
      } else {
        if constexpr (kKey4) kc[0][0] = *reinterpret_cast<const uint32_t*>(pg + 64 * 256 + row * 32 + 4 * c8);
        else kc[0] = *reinterpret_cast<const u32x2*>(pg + 64 * 256 + row * 64 + 8 * c8);
        s[8] = meta[kKeyScales + row * 8 + c8];
      }
    }
  }
  // Stepwise commit: step 2c converts the first half of 16-byte chunk c, step
  // 2c+1 the second half and stores the chunk (chunk 8 of a pass is the key).
  static constexpr int kStoreSteps = 18 * kPass;
  u32x2 part;
  template <int I>
  __device__ __forceinline__ void store_step(char* lds_buf) {
    constexpr int kcx = I / 2, p = kcx / 9, k = kcx % 9;
    u32x2 cur;
    if constexpr (k < 8) {
      const _Float16 sh = (_Float16)s[9 * p + k], zh = zero_h(8 * p + k, s[9 * p + k]);
      const half2v s2 = {sh, sh}, z2 = {zh, zh};
      const uint32_t w = n[8 * p + k];
      constexpr int j0 = 2 * (I % 2);
      cur = u32x2{nib2(w, j0, s2, z2), nib2(w, j0 + 1, s2, z2)};
    } else {
      const _Float16 kh = (_Float16)s[9 * p + 8];
      const half2v k2 = {kh, kh};
      if constexpr (kKey4) {
        const half2v z0 = {(_Float16)0.0f, (_Float16)0.0f};
        const uint32_t w = kc[p][0];
        constexpr int j0 = 2 * (I % 2);
        cur = u32x2{nib2(w, j0, k2, z0), nib2(w, j0 + 1, k2, z0)};
      } else {
        cur = int8x4_to_f16(kc[p][I % 2], k2);
      }
    }
    if constexpr (I % 2 == 0) {
      part = cur;
    } else {
      *reinterpret_cast<u32x4*>(lds_buf + swz<kSwz>(ltid<kTid0>() >> 3, ltid<kTid0>() & 7) + 32 * p * kRowLds + 128 * k) =
          u32x4{part[0], part[1], cur[0], cur[1]};
    }
  }
  __device__ __forceinline__ void commit(char* lds_buf) {
    const int tok = ltid<kTid0>() >> 3;
    char* dst = lds_buf + swz<kSwz>(tok, ltid<kTid0>() & 7);
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const _Float16 sh = (_Float16)s[9 * p + k], zh = zero_h(8 * p + k, s[9 * p + k]);
        const half2v s2 = {sh, sh}, z2 = {zh, zh};
        const uint32_t w = n[8 * p + k];
        u32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = nib2(w, j, s2, z2);
        *reinterpret_cast<u32x4*>(dst + 32 * p * kRowLds + 128 * k) = v;
      }
      const _Float16 kh = (_Float16)s[9 * p + 8];
      const half2v k2 = {kh, kh};
      if constexpr (kKey4) {
        const half2v z0 = {(_Float16)0.0f, (_Float16)0.0f};
        const uint32_t w = kc[p][0];
        *reinterpret_cast<u32x4*>(dst + 32 * p * kRowLds + 128 * 8) =
            u32x4{nib2(w, 0, k2, z0), nib2(w, 1, k2, z0), nib2(w, 2, k2, z0), nib2(w, 3, k2, z0)};
      } else {
        const u32x2 lo = int8x4_to_f16(kc[p][0], k2), hi = int8x4_to_f16(kc[p][1], k2);
        *reinterpret_cast<u32x4*>(dst + 32 * p * kRowLds + 128 * 8) = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Wide loaders of the 16-head kernel's staging waves (64-token tiles, 256
// threads): four threads per token, each loading 16-byte pieces, so that a tile
// takes a third of the load instructions of the loaders above (their narrow
// code, scale and zero loads made the staging waves issue-bound).  Thread t owns
// bytes 16 c4 + 64 i of each code row of token wide_tok(t), c4 = t % 4.  The
// values written to LDS are the same as the loaders above write.
//
// A wave covers 16 tokens; its 4-thread groups alternate between tokens r and
// r + 8, whose swizzle keys differ in their low bit, so that the eight threads
// of two neighbouring groups store into complementary halves of a 128-byte bank
// row (tokens r and r + 1 share a key and would collide).
template <int kTid0>
__device__ __forceinline__ int wide_tok() {
  const int t = ltid<kTid0>(), g = (t >> 2) & 15;
  return 16 * (t >> 6) + (g >> 1) + 8 * (g & 1);
}

// Eight packed nibbles (byte b: element 2b in its low nibble, 2b + 1 in its high
// one) -> eight fp16 values (q - 8) * s + z8, as four fp16 pairs, where z8 is
// the zero point plus 8 s (near the group's midpoint, see LoaderInt4Reg::nib2).
// Byte permutes place each nibble under the constant 0x64 high byte (fp16
// 1024 + q, exactly).  Symmetric INT4 (kSym): (q - 8) * s, no zero point.
template <bool kSym = false>
__device__ __forceinline__ u32x4 nib8_to_f16(uint32_t w, half2v s2, half2v z2) {
  const uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;
  const uint32_t x0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);   // lo.b0 hi.b0 lo.b1 hi.b1
  const uint32_t x1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);   // lo.b2 hi.b2 lo.b3 hi.b3
  // Each pair is formed in a scalar: hipcc's __builtin_bit_cast of a vector
  // element (r[j]) reads element 0 whatever the index.
  constexpr float kBias = -1032.0f;
  const half2v bias = {(_Float16)kBias, (_Float16)kBias};
  auto cv = [&](uint32_t h) {
    const half2v q = __builtin_bit_cast(half2v, h) + bias;
    if constexpr (kSym) return __builtin_bit_cast(uint32_t, q * s2);
    else return __builtin_bit_cast(uint32_t, q * s2 + z2);
  };
  return u32x4{cv(__builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u)), cv(__builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u)),
               cv(__builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u)), cv(__builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u))};
}

typedef float floatx2 __attribute__((ext_vector_type(2)));

// Loads written as inline assembly whose destination is tied to the register
// that held the previous tile ("+v"), for the staging waves of the 16-head
// kernel.  With compiler-visible loads, the register allocator kept the two
// alternating tiles in different registers from one pass of the loop to the
// next and copied them at the back edge; each copy waited for its load, so a
// load issued two steps ahead was in practice waited for one step ahead.  The
// compiler does not count these loads: their users wait with wait_vm<> and then
// settle() the registers (an empty asm that reads and writes them), so that no
// use moves above the wait.
template <int kOff>
__device__ __forceinline__ void asm_ld16_nt(u32x4& r, const void* p) {
  asm volatile("global_load_dwordx4 %0, %1, off offset:%2 nt" : "+v"(r) : "v"(p), "n"(kOff));
}
template <int kOff>
__device__ __forceinline__ void asm_ld16(floatx4& r, const void* p) {
  asm volatile("global_load_dwordx4 %0, %1, off offset:%2" : "+v"(r) : "v"(p), "n"(kOff));
}
template <int kOff, class T>
__device__ __forceinline__ void asm_ld8(T& r, const void* p) {
  static_assert(sizeof(T) == 8, "8-byte register pair");
  asm volatile("global_load_dwordx2 %0, %1, off offset:%2" : "+v"(r) : "v"(p), "n"(kOff));
}
template <int kOff>
__device__ __forceinline__ void asm_ld4(float& r, const void* p) {
  asm volatile("global_load_dword %0, %1, off offset:%2" : "+v"(r) : "v"(p), "n"(kOff));
}
template <class T>
__device__ __forceinline__ void settle(T& r) { asm volatile("" : "+v"(r)); }

// Value of x in lane kLane of this lane's quad (lanes 4q .. 4q + 3), by DPP.
template <int kLane>
__device__ __forceinline__ float quad_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), kLane * 0x55, 0xf, 0xf, false));
}

// 4 x 4 transpose within a quad: lane r (= r) of the quad returns
// (a_0[r], a_1[r], a_2[r], a_3[r]), a_k being lane k's argument.  Two exchange
// rounds, with partner r ^ 1 and then r ^ 2.
__device__ __forceinline__ floatx4 quad_transpose(floatx4 a, int r) {
  auto xchg = [](float v, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), decltype(ctrl)::value, 0xf, 0xf, false));
  };
  const bool r0 = r & 1, r1 = r & 2;
  floatx4 c;
#pragma unroll
  for (int p = 0; p < 2; ++p) {       // c[k] = a from lane (r & ~1) | (k & 1), component (k & ~1) | (r & 1)
    const float recv = xchg(r0 ? a[2 * p] : a[2 * p + 1], std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
    c[2 * p] = r0 ? recv : a[2 * p];
    c[2 * p + 1] = r0 ? a[2 * p + 1] : recv;
  }
  floatx4 d;
#pragma unroll
  for (int q = 0; q < 2; ++q) {       // d[k] = c from lane (r & ~2) | (k & 2), component (k & ~2) | (r & 2)
    const float recv = xchg(r1 ? c[q] : c[q + 2], std::integral_constant<int, 0x4E>{});       // quad_perm [2,3,0,1]
    d[q] = r1 ? recv : c[q];
    d[q + 2] = r1 ? c[q + 2] : recv;
  }
  return d;
}

// bf16 for the 16-head kernel's staging waves: the row mapping of LoaderBf16Reg
// (eight threads per token, two 32-token passes), with tied assembly loads.
template <int kSwz, int kTid0>
struct LoaderBf16Wide {
  __device__ __forceinline__ void set_lo(int) {}   // rows below a bound are masked by the scores instead
  static constexpr int kLoads = 18;      // load instructions per tile
  u32x4 r[18] = {};

  __device__ __forceinline__ bool issue(const DecodeArgs& a, int64_t page, int t0, int t_end) {
    const int tok = ltid<kTid0>() >> 3;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const bool ok = page >= 0 && t0 + 32 * p + tok < t_end;
      const uint8_t* src = page_base(a, page, ok, kBlock * kRowBytesBf16) +
                           ((t0 % kBlock) + 32 * p + tok) * kRowBytesBf16 + 16 * (ltid<kTid0>() & 7);
      asm_ld16_nt<0>(r[9 * p + 0], src);
      asm_ld16_nt<128>(r[9 * p + 1], src);
      asm_ld16_nt<256>(r[9 * p + 2], src);
      asm_ld16_nt<384>(r[9 * p + 3], src);
      asm_ld16_nt<512>(r[9 * p + 4], src);
      asm_ld16_nt<640>(r[9 * p + 5], src);
      asm_ld16_nt<768>(r[9 * p + 6], src);
      asm_ld16_nt<896>(r[9 * p + 7], src);
      asm_ld16_nt<1024>(r[9 * p + 8], src);
    }
    return page >= 0;
  }
  __device__ __forceinline__ void settle_all() {
#pragma unroll
    for (int k = 0; k < 18; ++k) settle(r[k]);
  }
  __device__ __forceinline__ void commit(char* lds_buf) {
    const int tok = ltid<kTid0>() >> 3;
    char* dst = lds_buf + swz<kSwz>(tok, ltid<kTid0>() & 7);
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int k = 0; k < 9; ++k)
        *reinterpret_cast<u32x4*>(dst + 32 * p * kRowLds + 128 * k) = bf16x8_to_f16x8(r[9 * p + k]);
  }
  // commit() and then issue() of the next tile, interleaved: each chunk's
  // registers are reloaded right after they are stored, so that the loads
  // leave while the rest of the tile is converted (a wave that issues them in
  // one burst stalls while the CU's load queue is full).
  template <int I>
  __device__ __forceinline__ void chunk(char* dst, const uint8_t* src0, const uint8_t* src1) {
    constexpr int p = I / 9, k = I % 9;
    *reinterpret_cast<u32x4*>(dst + 32 * p * kRowLds + 128 * k) = bf16x8_to_f16x8(r[I]);
    __builtin_amdgcn_sched_barrier(0);     // the reload may not overtake the conversion of the same registers
    asm_ld16_nt<128 * k>(r[I], p == 0 ? src0 : src1);
    if constexpr (I + 1 < 18) chunk<I + 1>(dst, src0, src1);
  }
  __device__ __forceinline__ void commit_issue(char* lds_buf, const DecodeArgs& a, int64_t page, int t0, int t_end) {
    const int tok = ltid<kTid0>() >> 3;
    const uint8_t* src[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const bool ok = page >= 0 && t0 + 32 * p + tok < t_end;
      src[p] = page_base(a, page, ok, kBlock * kRowBytesBf16) + ((t0 % kBlock) + 32 * p + tok) * kRowBytesBf16 +
               16 * (ltid<kTid0>() & 7);
    }
    chunk<0>(lds_buf + swz<kSwz>(tok, ltid<kTid0>() & 7), src[0], src[1]);
  }
};

// INT8 (page: [64][576] codes | [64][16] f32 latent scales | [64][8] f32 key
// scales).  Piece i < 8 holds latent codes 64 i + 16 c4 .. +15, one 32-code
// block (c4 / 2 + 2 i); piece 8 the key codes 16 c4 .. +15, key blocks 2 c4 and
// 2 c4 + 1.  Its two 8-code halves are LDS chunks 2 c4 and 2 c4 + 1 of 128-byte
// group i.  The four threads of a token (one quad of lanes) load its 16 latent
// scales as four 16-byte pieces and pass them round by DPP: one load instead of
// eight 4-byte ones, since load instructions, not bytes, pace the staging.
// Per-token INT8 (kTok1): the token's one latent scale is a single 4-byte load
// (every thread of the token loads it), no DPP.  FP8 per token (kFp8, with
// kTok1): the same page with e4m3 codes.
template <int kSwz, int kTid0, bool kTok1 = false, bool kFp8 = false>
struct LoaderInt8Wide {
  __device__ __forceinline__ void set_lo(int) {}   // rows below a bound are masked by the scores instead
  static constexpr int kPage = kBlock * (kTok1 ? 612 : 672);
  static constexpr int kLoads = 11;      // load instructions per tile
  static constexpr int kKeyScales = 64 * 576 + (kTok1 ? 64 * 4 : 64 * 64);   // byte offset of the key scales
  u32x4 c[9] = {};
  floatx4 sv = {};           // latent scales 4 c4 .. 4 c4 + 3 of the token
  float st = 0.f;            // per token: the token's latent scale
  floatx2 ks = {};

  __device__ __forceinline__ bool issue(const DecodeArgs& a, int64_t page, int t0, int t_end) {
    const int tok = wide_tok<kTid0>(), c4 = ltid<kTid0>() & 3;
    const bool ok = page >= 0 && t0 + tok < t_end;
    const int row = (t0 % kBlock) + tok;
    const uint8_t* pg = page_base(a, page, ok, kPage);
    const uint8_t* codes = pg + row * 576 + 16 * c4;
    asm_ld16_nt<0>(c[0], codes);
    asm_ld16_nt<64>(c[1], codes);
    asm_ld16_nt<128>(c[2], codes);
    asm_ld16_nt<192>(c[3], codes);
    asm_ld16_nt<256>(c[4], codes);
    asm_ld16_nt<320>(c[5], codes);
    asm_ld16_nt<384>(c[6], codes);
    asm_ld16_nt<448>(c[7], codes);
    asm_ld16_nt<512>(c[8], codes);
    if constexpr (kTok1) asm_ld4<0>(st, pg + 64 * 576 + row * 4);
    else asm_ld16<0>(sv, pg + 64 * 576 + row * 64 + 16 * c4);
    asm_ld8<0>(ks, pg + kKeyScales + row * 32 + 8 * c4);
    return page >= 0;
  }
  __device__ __forceinline__ void settle_all() {
#pragma unroll
    for (int i = 0; i < 9; ++i) settle(c[i]);
    if constexpr (kTok1) settle(st);
    else settle(sv);
    settle(ks);
  }
  // Scale of piece i < 8, block b = c4 / 2 + 2 i: component b % 4 of quad lane b / 4 = i / 2.
  template <int I>
  __device__ __forceinline__ float scale(bool upper) const {
    if constexpr (kTok1) return st;
    const float lo = quad_bcast<I / 2>(sv[2 * (I % 2)]), hi = quad_bcast<I / 2>(sv[2 * (I % 2) + 1]);
    return upper ? hi : lo;
  }
  template <int I>
  __device__ __forceinline__ void commit_piece(char* d0, char* d1, bool upper) {
    float f0, f1;
    if constexpr (I < 8) {
      f0 = f1 = scale<I>(upper);
    } else {
      f0 = ks[0];
      f1 = ks[1];
    }
    const _Float16 s0 = code_scale_h<kFp8>(f0), s1 = code_scale_h<kFp8>(f1);
    const u32x2 a0 = codes4_to_f16_perm<kFp8>(c[I][0], half2v{s0, s0}), a1 = codes4_to_f16_perm<kFp8>(c[I][1], half2v{s0, s0});
    const u32x2 b0 = codes4_to_f16_perm<kFp8>(c[I][2], half2v{s1, s1}), b1 = codes4_to_f16_perm<kFp8>(c[I][3], half2v{s1, s1});
    *reinterpret_cast<u32x4*>(d0 + 128 * I) = u32x4{a0[0], a0[1], a1[0], a1[1]};
    *reinterpret_cast<u32x4*>(d1 + 128 * I) = u32x4{b0[0], b0[1], b1[0], b1[1]};
  }
  __device__ __forceinline__ void commit(char* lds_buf) {
    const int tok = wide_tok<kTid0>(), c4 = ltid<kTid0>() & 3;
    char* d0 = lds_buf + swz<kSwz>(tok, 2 * c4);
    char* d1 = lds_buf + swz<kSwz>(tok, 2 * c4 + 1);
    const bool upper = c4 >= 2;
    commit_piece<0>(d0, d1, upper);
    commit_piece<1>(d0, d1, upper);
    commit_piece<2>(d0, d1, upper);
    commit_piece<3>(d0, d1, upper);
    commit_piece<4>(d0, d1, upper);
    commit_piece<5>(d0, d1, upper);
    commit_piece<6>(d0, d1, upper);
    commit_piece<7>(d0, d1, upper);
    commit_piece<8>(d0, d1, upper);
  }
  // commit() and then issue() of the next tile, interleaved (as LoaderBf16Wide):
  // each piece's codes are reloaded right after it is converted and stored; the
  // scales, which every piece uses, last.  The loads keep issue()'s order.
  template <int I>
  __device__ __forceinline__ void piece(char* d0, char* d1, bool upper, const uint8_t* codes) {
    commit_piece<I>(d0, d1, upper);
    __builtin_amdgcn_sched_barrier(0);     // the reload may not overtake the conversion of the same registers
    asm_ld16_nt<64 * I>(c[I], codes);
    if constexpr (I + 1 < 9) piece<I + 1>(d0, d1, upper, codes);
  }
  __device__ __forceinline__ void commit_issue(char* lds_buf, const DecodeArgs& a, int64_t page, int t0, int t_end) {
    const int tok = wide_tok<kTid0>(), c4 = ltid<kTid0>() & 3;
    const bool ok = page >= 0 && t0 + tok < t_end;
    const int row = (t0 % kBlock) + tok;
    const uint8_t* pg = page_base(a, page, ok, kPage);
    piece<0>(lds_buf + swz<kSwz>(tok, 2 * c4), lds_buf + swz<kSwz>(tok, 2 * c4 + 1), c4 >= 2, pg + row * 576 + 16 * c4);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kTok1) asm_ld4<0>(st, pg + 64 * 576 + row * 4);
    else asm_ld16<0>(sv, pg + 64 * 576 + row * 64 + 16 * c4);
    asm_ld8<0>(ks, pg + kKeyScales + row * 32 + 8 * c4);
  }
};

// INT4 (page: [64][256] latent nibbles | [64][64] int8 key codes | [64][16] f32
// scales | [64][16] f32 zeros | [64][8] f32 key scales).  Piece i < 4 holds the
// 32 latent values 32 c4 + 128 i .. +31, one block (c4 + 4 i); its 16-byte
// chunks j = 0..3 are chunks 4 (c4 % 2) + j of 128-byte group 2 i + c4 / 2.
// Threads c4 >= 2 write their chunks in the order j ^ 2, so that the four
// threads of a token write four different LDS bank groups at every store.  The
// key piece (16 codes at 16 c4) goes to chunks 2 c4, 2 c4 + 1 of group 8.
// kKey4 (with kSym): the RoPE key as symmetric INT4, 16 nibbles (two 8-groups)
// per thread in one 8-byte load.
template <int kSwz, int kTid0, bool kSym = false, bool kKey4 = false>
struct LoaderInt4Wide {
  __device__ __forceinline__ void set_lo(int) {}   // rows below a bound are masked by the scores instead
  static constexpr int kLoads = kSym ? 7 : 8;   // load instructions per tile
  static constexpr int kPage = kBlock * (kKey4 ? 384 : (kSym ? 416 : 480));
  static constexpr int kKeyScales = kSym ? 64 * 64 : 2 * 64 * 64;   // byte offset of the key scales after the scales
  u32x4 n[4] = {};
  floatx4 sq = {}, zq = {};  // scales / zeros 4 c4 .. 4 c4 + 3 of the token (transposed in commit)
  u32x4 kc = {};
  u32x2 kn = {};             // kKey4: key nibbles 16 c4 .. 16 c4 + 15
  floatx2 ks = {};

  __device__ __forceinline__ bool issue(const DecodeArgs& a, int64_t page, int t0, int t_end) {
    const int tok = wide_tok<kTid0>(), c4 = ltid<kTid0>() & 3;
    const bool ok = page >= 0 && t0 + tok < t_end;
    const int row = (t0 % kBlock) + tok;
    const uint8_t* pg = page_base(a, page, ok, kPage);
    const uint8_t* nib = pg + row * 256 + 16 * c4;
    asm_ld16_nt<0>(n[0], nib);
    asm_ld16_nt<64>(n[1], nib);
    asm_ld16_nt<128>(n[2], nib);
    asm_ld16_nt<192>(n[3], nib);
    if constexpr (kKey4) asm_ld8<0>(kn, pg + 64 * 256 + row * 32 + 8 * c4);
    else asm_ld16_nt<0>(kc, pg + 64 * 256 + row * 64 + 16 * c4);
    const uint8_t* meta = pg + 64 * 256 + 64 * (kKey4 ? 32 : 64);
    asm_ld16<0>(sq, meta + row * 64 + 16 * c4);
    if constexpr (!kSym) asm_ld16<0>(zq, meta + 64 * 64 + row * 64 + 16 * c4);
    asm_ld8<0>(ks, meta + kKeyScales + row * 32 + 8 * c4);
    return page >= 0;
  }
  __device__ __forceinline__ void settle_all() {
#pragma unroll
    for (int i = 0; i < 4; ++i) settle(n[i]);
    settle(sq);
    if constexpr (!kSym) settle(zq);
    if constexpr (kKey4) settle(kn);
    else settle(kc);
    settle(ks);
  }
  __device__ __forceinline__ void commit(char* lds_buf) {
    const int tok = wide_tok<kTid0>(), c4 = ltid<kTid0>() & 3;
    const bool swap = c4 >= 2;
    // All-ones for swapping threads; opaque, so that the choice below stays a
    // bitwise blend (one v_bfi) instead of becoming a runtime array index.
    uint32_t blend = swap ? ~0u : 0u;
    asm volatile("" : "+v"(blend));
    char* dst[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = lds_buf + swz<kSwz>(tok, 4 * (c4 & 1) + (j ^ (swap ? 2 : 0))) + 128 * (c4 >> 1);
    // Block c4 + 4 i's scale is component c4 of quad lane i's sq: a 4 x 4
    // transpose within the quad.
    const floatx4 st = quad_transpose(sq, c4);
    floatx4 zt = floatx4{};
    if constexpr (!kSym) zt = quad_transpose(zq, c4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 sh = (_Float16)st[i], zh = kSym ? (_Float16)0.0f : (_Float16)fmaf(8.0f, st[i], zt[i]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = (n[i][j] & ~blend) | (n[i][j ^ 2] & blend);
        *reinterpret_cast<u32x4*>(dst[j] + 256 * i) = nib8_to_f16<kSym>(w, half2v{sh, sh}, half2v{zh, zh});
      }
    }
    const _Float16 k0 = (_Float16)ks[0], k1 = (_Float16)ks[1];
    if constexpr (kKey4) {
      const half2v z0 = {(_Float16)0.0f, (_Float16)0.0f};
      *reinterpret_cast<u32x4*>(lds_buf + swz<kSwz>(tok, 2 * c4) + 128 * 8) = nib8_to_f16<true>(kn[0], half2v{k0, k0}, z0);
      *reinterpret_cast<u32x4*>(lds_buf + swz<kSwz>(tok, 2 * c4 + 1) + 128 * 8) =
          nib8_to_f16<true>(kn[1], half2v{k1, k1}, z0);
    } else {
      const u32x2 a0 = int8x4_to_f16_perm(kc[0], half2v{k0, k0}), a1 = int8x4_to_f16_perm(kc[1], half2v{k0, k0});
      const u32x2 b0 = int8x4_to_f16_perm(kc[2], half2v{k1, k1}), b1 = int8x4_to_f16_perm(kc[3], half2v{k1, k1});
      *reinterpret_cast<u32x4*>(lds_buf + swz<kSwz>(tok, 2 * c4) + 128 * 8) = u32x4{a0[0], a0[1], a1[0], a1[1]};
      *reinterpret_cast<u32x4*>(lds_buf + swz<kSwz>(tok, 2 * c4 + 1) + 128 * 8) = u32x4{b0[0], b0[1], b1[0], b1[1]};
    }
  }
};

// INT8 per channel over 32-token blocks, closed blocks (page: [64][512] latent
// codes | [64][64] key codes | [2][512] f32 channel scales | [64][8] f32 key
// scales | overflow).  Threads are laid out down the channels so that each one
// needs only 16 of the block's channel scales: thread t owns the 16-channel
// piece p = t % 32 (LDS chunks 2p, 2p + 1) of the 8 tokens 8 (t / 32) + m of
// one block (tile rows 0..31 are block 0, 32..63 block 1), and the key piece
// t % 4 (16 key codes, groups 2 (t % 4) and 2 (t % 4) + 1) of token t / 4.
template <int kSwz, int kTid0>
struct LoaderInt8cWide {
  static constexpr int kLoads = 14;      // load instructions per tile
  u32x4 c[8] = {};
  floatx4 sv[4] = {};
  u32x4 kc = {};
  floatx2 ks = {};
  __device__ __forceinline__ void set_lo(int) {}

  __device__ __forceinline__ bool issue(const DecodeArgs& a, int64_t page, int t0, int t_end) {
    const int lt = ltid<kTid0>(), p = lt & 31, tg = lt >> 5;
    const int tok0 = 8 * tg;
#define MLA_I8C_ROW(m)                                                                                     \
    asm_ld16_nt<0>(c[m], page_base(a, page, page >= 0 && t0 + tok0 + (m) < t_end, kPageInt8c) +              \
                             (tok0 + (m)) * 512 + 16 * p)
    MLA_I8C_ROW(0);
    MLA_I8C_ROW(1);
    MLA_I8C_ROW(2);
    MLA_I8C_ROW(3);
    MLA_I8C_ROW(4);
    MLA_I8C_ROW(5);
    MLA_I8C_ROW(6);
    MLA_I8C_ROW(7);
#undef MLA_I8C_ROW
    // a block past t_end may hold no scales yet: read the zero page's (the codes are zero too)
    const uint8_t* sc = page_base(a, page, page >= 0 && t0 + 32 * (tg >> 2) < t_end, kPageInt8c) + kI8cScales +
                        (tg >> 2) * 2048 + 64 * p;
    asm_ld16<0>(sv[0], sc);
    asm_ld16<16>(sv[1], sc);
    asm_ld16<32>(sv[2], sc);
    asm_ld16<48>(sv[3], sc);
    const int ktok = lt >> 2, kq = lt & 3;
    const uint8_t* kp = page_base(a, page, page >= 0 && t0 + ktok < t_end, kPageInt8c);
    asm_ld16_nt<0>(kc, kp + kI8cKeyCodes + ktok * 64 + 16 * kq);
    asm_ld8<0>(ks, kp + kI8cKeyScales + ktok * 32 + 8 * kq);
    return page >= 0;
  }
  __device__ __forceinline__ void settle_all() {
#pragma unroll
    for (int i = 0; i < 8; ++i) settle(c[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) settle(sv[i]);
    settle(kc);
    settle(ks);
  }
  __device__ __forceinline__ void commit(char* lds_buf) {
    const int lt = ltid<kTid0>(), p = lt & 31, tok0 = 8 * (lt >> 5);
    // fp16 scale pairs of channels (2j, 2j + 1) of the piece
    half2v s2[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s2[j] = half2v{(_Float16)sv[j >> 1][2 * (j & 1)], (_Float16)sv[j >> 1][2 * (j & 1) + 1]};
    const half2v bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      uint32_t h[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t u = c[m][d] ^ 0x80808080u;
        const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);   // codes 4d, 4d + 1
        const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);   // codes 4d + 2, 4d + 3
        h[2 * d] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2v, lo) + bias) * s2[2 * d]);
        h[2 * d + 1] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2v, hi) + bias) * s2[2 * d + 1]);
      }
      *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(tok0 + m, 2 * p)) = u32x4{h[0], h[1], h[2], h[3]};
      *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(tok0 + m, 2 * p + 1)) = u32x4{h[4], h[5], h[6], h[7]};
    }
    const int ktok = lt >> 2, kq = lt & 3;
    const _Float16 k0 = (_Float16)ks[0], k1 = (_Float16)ks[1];
    const u32x2 a0 = int8x4_to_f16_perm(kc[0], half2v{k0, k0}), a1 = int8x4_to_f16_perm(kc[1], half2v{k0, k0});
    const u32x2 b0 = int8x4_to_f16_perm(kc[2], half2v{k1, k1}), b1 = int8x4_to_f16_perm(kc[3], half2v{k1, k1});
    *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(ktok, 64 + 2 * kq)) = u32x4{a0[0], a0[1], a1[0], a1[1]};
    *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(ktok, 64 + 2 * kq + 1)) = u32x4{b0[0], b0[1], b1[0], b1[1]};
  }
  // commit() and then issue() of the next tile, interleaved (as LoaderInt8Wide):
  // the channel scales are taken into registers first, each code row is
  // reloaded right after it is stored, then the scales and the RoPE key.  The
  // loads keep issue()'s order.
  template <int M>
  __device__ __forceinline__ void row(char* lds_buf, const half2v (&s2)[8], const DecodeArgs& a, int64_t page, int t0,
                                      int t_end) {
    const int lt = ltid<kTid0>(), p = lt & 31, tok0 = 8 * (lt >> 5);
    const half2v bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    uint32_t h[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t u = c[M][d] ^ 0x80808080u;
      const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
      const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
      h[2 * d] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2v, lo) + bias) * s2[2 * d]);
      h[2 * d + 1] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2v, hi) + bias) * s2[2 * d + 1]);
    }
    *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(tok0 + M, 2 * p)) = u32x4{h[0], h[1], h[2], h[3]};
    *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(tok0 + M, 2 * p + 1)) = u32x4{h[4], h[5], h[6], h[7]};
    __builtin_amdgcn_sched_barrier(0);     // the reload may not overtake the conversion of the same registers
    asm_ld16_nt<0>(c[M], page_base(a, page, page >= 0 && t0 + tok0 + M < t_end, kPageInt8c) + (tok0 + M) * 512 + 16 * p);
    if constexpr (M + 1 < 8) row<M + 1>(lds_buf, s2, a, page, t0, t_end);
  }
  __device__ __forceinline__ void commit_issue(char* lds_buf, const DecodeArgs& a, int64_t page, int t0, int t_end) {
    const int lt = ltid<kTid0>(), p = lt & 31, tg = lt >> 5;
    half2v s2[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s2[j] = half2v{(_Float16)sv[j >> 1][2 * (j & 1)], (_Float16)sv[j >> 1][2 * (j & 1) + 1]};
    row<0>(lds_buf, s2, a, page, t0, t_end);
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* sc = page_base(a, page, page >= 0 && t0 + 32 * (tg >> 2) < t_end, kPageInt8c) + kI8cScales +
                        (tg >> 2) * 2048 + 64 * p;
    asm_ld16<0>(sv[0], sc);
    asm_ld16<16>(sv[1], sc);
    asm_ld16<32>(sv[2], sc);
    asm_ld16<48>(sv[3], sc);
    const int ktok = lt >> 2, kq = lt & 3;
    const _Float16 k0 = (_Float16)ks[0], k1 = (_Float16)ks[1];
    const u32x2 a0 = int8x4_to_f16_perm(kc[0], half2v{k0, k0}), a1 = int8x4_to_f16_perm(kc[1], half2v{k0, k0});
    const u32x2 b0 = int8x4_to_f16_perm(kc[2], half2v{k1, k1}), b1 = int8x4_to_f16_perm(kc[3], half2v{k1, k1});
    *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(ktok, 64 + 2 * kq)) = u32x4{a0[0], a0[1], a1[0], a1[1]};
    *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(ktok, 64 + 2 * kq + 1)) = u32x4{b0[0], b0[1], b1[0], b1[1]};
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* kp = page_base(a, page, page >= 0 && t0 + ktok < t_end, kPageInt8c);
    asm_ld16_nt<0>(kc, kp + kI8cKeyCodes + ktok * 64 + 16 * kq);
    asm_ld8<0>(ks, kp + kI8cKeyScales + ktok * 32 + 8 * kq);
  }
};

// The open block of the per-channel INT8 format: latent rows in bf16, channels
// 0..255 in the row's own code row and 256..511 in overflow row (row % 32); the
// RoPE key INT8 as for closed rows.  Thread t takes token t / 4: latent
// channels 128 (t % 4) .. +127 (16 chunks of 8) and key piece t % 4.  Rows
// below t_lo (closed rows of the same page) and past t_end read the zero page.
template <int kSwz, int kTid0>
struct LoaderInt8cOpenWide {
  static constexpr int kLoads = 18;      // load instructions per tile
  u32x4 v[16] = {};
  u32x4 kc = {};
  floatx2 ks = {};
  int t_lo = 0;
  __device__ __forceinline__ void set_lo(int lo) { t_lo = lo; }

  __device__ __forceinline__ bool issue(const DecodeArgs& a, int64_t page, int t0, int t_end) {
    const int lt = ltid<kTid0>(), tok = lt >> 2, c4 = lt & 3;
    const bool ok = page >= 0 && t0 + tok < t_end && t0 + tok >= t_lo;
    const uint8_t* pg = page_base(a, page, ok, kPageInt8c);
    // c4 = 0, 1: channels < 256 in the token's code row; c4 = 2, 3: its overflow row
    const uint8_t* src = pg + (c4 < 2 ? tok * 512 + 256 * c4 : kI8cOverflow + (tok % 32) * 512 + 256 * (c4 - 2));
    asm_ld16_nt<0>(v[0], src);
    asm_ld16_nt<16>(v[1], src);
    asm_ld16_nt<32>(v[2], src);
    asm_ld16_nt<48>(v[3], src);
    asm_ld16_nt<64>(v[4], src);
    asm_ld16_nt<80>(v[5], src);
    asm_ld16_nt<96>(v[6], src);
    asm_ld16_nt<112>(v[7], src);
    asm_ld16_nt<128>(v[8], src);
    asm_ld16_nt<144>(v[9], src);
    asm_ld16_nt<160>(v[10], src);
    asm_ld16_nt<176>(v[11], src);
    asm_ld16_nt<192>(v[12], src);
    asm_ld16_nt<208>(v[13], src);
    asm_ld16_nt<224>(v[14], src);
    asm_ld16_nt<240>(v[15], src);
    asm_ld16_nt<0>(kc, pg + kI8cKeyCodes + tok * 64 + 16 * c4);
    asm_ld8<0>(ks, pg + kI8cKeyScales + tok * 32 + 8 * c4);
    return page >= 0;
  }
  __device__ __forceinline__ void settle_all() {
#pragma unroll
    for (int i = 0; i < 16; ++i) settle(v[i]);
    settle(kc);
    settle(ks);
  }
  __device__ __forceinline__ void commit(char* lds_buf) {
    const int lt = ltid<kTid0>(), tok = lt >> 2, c4 = lt & 3;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(tok, 16 * c4 + i)) = bf16x8_to_f16x8(v[i]);
    const _Float16 k0 = (_Float16)ks[0], k1 = (_Float16)ks[1];
    const u32x2 a0 = int8x4_to_f16_perm(kc[0], half2v{k0, k0}), a1 = int8x4_to_f16_perm(kc[1], half2v{k0, k0});
    const u32x2 b0 = int8x4_to_f16_perm(kc[2], half2v{k1, k1}), b1 = int8x4_to_f16_perm(kc[3], half2v{k1, k1});
    *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(tok, 64 + 2 * c4)) = u32x4{a0[0], a0[1], a1[0], a1[1]};
    *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(tok, 64 + 2 * c4 + 1)) = u32x4{b0[0], b0[1], b1[0], b1[1]};
  }
  // commit() and then issue() of the next tile, interleaved (as LoaderBf16Wide).
  template <int I>
  __device__ __forceinline__ void chunk(char* lds_buf, const uint8_t* src) {
    const int tok = ltid<kTid0>() >> 2, c4 = ltid<kTid0>() & 3;
    *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(tok, 16 * c4 + I)) = bf16x8_to_f16x8(v[I]);
    __builtin_amdgcn_sched_barrier(0);     // the reload may not overtake the conversion of the same registers
    asm_ld16_nt<16 * I>(v[I], src);
    if constexpr (I + 1 < 16) chunk<I + 1>(lds_buf, src);
  }
  __device__ __forceinline__ void commit_issue(char* lds_buf, const DecodeArgs& a, int64_t page, int t0, int t_end) {
    const int lt = ltid<kTid0>(), tok = lt >> 2, c4 = lt & 3;
    const bool ok = page >= 0 && t0 + tok < t_end && t0 + tok >= t_lo;
    const uint8_t* pg = page_base(a, page, ok, kPageInt8c);
    chunk<0>(lds_buf, pg + (c4 < 2 ? tok * 512 + 256 * c4 : kI8cOverflow + (tok % 32) * 512 + 256 * (c4 - 2)));
    __builtin_amdgcn_sched_barrier(0);
    const _Float16 k0 = (_Float16)ks[0], k1 = (_Float16)ks[1];
    const u32x2 a0 = int8x4_to_f16_perm(kc[0], half2v{k0, k0}), a1 = int8x4_to_f16_perm(kc[1], half2v{k0, k0});
    const u32x2 b0 = int8x4_to_f16_perm(kc[2], half2v{k1, k1}), b1 = int8x4_to_f16_perm(kc[3], half2v{k1, k1});
    *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(tok, 64 + 2 * c4)) = u32x4{a0[0], a0[1], a1[0], a1[1]};
    *reinterpret_cast<u32x4*>(lds_buf + swz_chunk<kSwz>(tok, 64 + 2 * c4 + 1)) = u32x4{b0[0], b0[1], b1[0], b1[1]};
    __builtin_amdgcn_sched_barrier(0);
    asm_ld16_nt<0>(kc, pg + kI8cKeyCodes + tok * 64 + 16 * c4);
    asm_ld8<0>(ks, pg + kI8cKeyScales + tok * 32 + 8 * c4);
  }
};

// ===========================================================================
// H = 128
// ===========================================================================
// Per 32-token tile and wave w (4 waves, one work-group per work item):
//   scores   S^T[32 tok x 32 heads] for heads 32w..32w+31 over all 576 columns:
//            36 x mfma 32x32x16 (K fragments from the LDS tile, Q^T in VGPRs);
//   softmax  per head against a fixed reference max; P (fp16) is written to a
//            small LDS exchange buffer [128 heads][32 tokens];
//   values   O^T[128 features x 128 heads] for features 128w..128w+127:
//            32 x mfma 32x32x16 (V^T read transposed from the tile, P^T of all
//            heads from the exchange buffer).
// Splitting the value product by features rather than heads makes every wave
// read only its quarter of V; the LDS, not the matrix cores, is the scarce unit.
// The next tile is staged meanwhile: its rows sit in VGPRs (loaded one tile
// ahead), are widened to fp16 and written to the other LDS buffer between the
// value MFMAs; then the loads for the tile after it are issued.
constexpr int kTile128 = 32;
constexpr int kBuf128 = kTile128 * kRowLds;        // 36,864 B
constexpr int kPRow = 2 * kTile128;                // P exchange row: 32 tokens x fp16
constexpr int kPBuf = 128 * kPRow;                 // 8,192 B

struct H128Lane {
  uint32_t qk_off[4];     // score operand: row hl, chunk 2 k4 + g
  uint32_t pv_off[4];     // transposed value read: row 4 g + (gi >> 2) + 8 hi; [2 hi + parity]
  int g, hl;
  // P exchange: head hl's 16 bytes for token half j (head group 0).
  __device__ __forceinline__ uint32_t p_off(int j) const { return hl * kPRow + 16 * ((2 * j + g) ^ ((hl >> 2) & 3)); }
};

// Q^T of the first kQReg k-steps (16 columns each) stays in VGPRs; the last
// kQTail k-steps (128 latent columns and the 64 RoPE columns) of all 128 heads
// live in LDS, which leaves the VGPRs the tile pipeline needs.  Row h (256 B)
// holds q_abs[b][h][448..575], 16-byte chunk c stored at c ^ (h & 15), so the 16
// heads a lane group reads land in distinct banks.
constexpr int kQReg = 28, kQTail = kDk / 16 - kQReg;
constexpr int kQTailRow = kQTail * 32;                    // 256 B
constexpr int kQTailBytes = 128 * kQTailRow;              // 32,768 B
__device__ __forceinline__ uint32_t qtail_off(int h, int c) { return h * kQTailRow + 16 * (c ^ (h & 15)); }

// P exchange layout: row h (64 B) holds, for token half j and lane group g, the
// eight fp16 values lane (g, h % 32) of the owning wave computed, in the 16-byte
// chunk (2 j + g) ^ ((h >> 2) & 3) (the XOR keeps 16-lane accesses conflict free).
__device__ __forceinline__ H128Lane h128_lane() {
  H128Lane L;
  const int lane = threadIdx.x & 63;
  const int hl = lane & 31, g = lane >> 5, grp = lane >> 4, gi = lane & 15;
  L.g = g;
  L.hl = hl;
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) L.qk_off[k4] = swz<kSwz128>(hl, 2 * k4 + g);
#pragma unroll
  for (int hi = 0; hi < 2; ++hi) {
    const int pv_row = 4 * g + (gi >> 2) + 8 * hi;
#pragma unroll
    for (int par = 0; par < 2; ++par)
      L.pv_off[2 * hi + par] = swz<kSwz128>(pv_row, 4 * par + 2 * (grp & 1) + ((gi & 3) >> 1)) + 8 * (gi & 1);
  }
  return L;
}

// Score MFMA chain of one tile, as fenced steps: step ks issues MFMA ks and the
// K (and, for the last columns, Q^T) fragment reads kPf steps ahead.  kPf is as deep as the registers allow without
// spilling: a spill reload here would wait behind the tile loads in flight
// (vector-memory counters retire in order).
template <int kPf>
struct H128Scores {
  const char* buf;
  const char* qtail;
  const H128Lane& L;
  const half8 (&q)[kQReg];
  int hq;
  floatx16 sacc;
  half8 kb[kPf], qb[kPf];
  static constexpr int kSteps = kDk / 16;

  __device__ __forceinline__ half8 kread(int ks) const {
    return *reinterpret_cast<const half8*>(buf + L.qk_off[ks & 3] + 128 * (ks >> 2));
  }
  template <int KS>
  __device__ __forceinline__ void step() {
    if constexpr (KS < kQReg) sacc = mfma32x32x16(kb[KS % kPf], q[KS], sacc);
    else sacc = mfma32x32x16(kb[KS % kPf], qb[KS % kPf], sacc);
    constexpr int kn = KS + kPf;
    if constexpr (kn < kSteps) {
      kb[KS % kPf] = kread(kn);
      if constexpr (kn >= kQReg)
        qb[KS % kPf] = *reinterpret_cast<const half8*>(qtail + qtail_off(hq, 2 * (kn - kQReg) + L.g));
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (KS + 1 < kSteps) step<KS + 1>();
  }
  __device__ __forceinline__ floatx16 run() {
    __builtin_amdgcn_sched_barrier(0);
    sacc = floatx16{};
#pragma unroll
    for (int d = 0; d < kPf; ++d) kb[d] = kread(d);
    static_assert(kQReg >= kPf, "the first Q^T fragments come from VGPRs");
    __builtin_amdgcn_sched_barrier(0);
    step<0>();
    return sacc;
  }
};

// Scores and softmax of one tile for this wave's 32 heads.  kMode 0: fixed
// reference max per head, taken at its first non-empty tile (`overflow` is set
// when a later tile exceeds it by more than kTauFixed); kMode 1: scores only,
// m_ref becomes the exact max; kMode 2: against the exact max in m_ref.
// Returns P^T as the value product's B operand (p[j]: token half j).
template <int kMode, int kPf>
__device__ __forceinline__ void h128_scores(const char* buf, const char* qtail, const H128Lane& L,
                                            const half8 (&q)[kQReg], float& m_ref, float& l_sum,
                                            bool& overflow, int t0, int t_end, bool page_ok, float scale_log2,
                                            half8 (&p)[2]) {
  floatx16 sacc = H128Scores<kPf>{buf, qtail, L, q, 32 * (int)(threadIdx.x >> 6) + L.hl}.run();
#pragma unroll
  for (int r = 0; r < 16; ++r) sacc[r] *= scale_log2;
  if (!page_ok || t0 + kTile128 > t_end) {          // partial tile: mask the missing rows
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tt = t0 + 8 * (r >> 2) + 4 * L.g + (r & 3);
      if (!page_ok || tt >= t_end) sacc[r] = -INFINITY;
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
  mx = max_xor32(mx);                      // lanes l and l^32 hold the same head
  if (kMode == 1) {
    m_ref = fmaxf(m_ref, mx);
    return;
  }
  if (kMode == 0) {
    if (m_ref == -INFINITY) m_ref = mx;    // first non-empty tile: nothing accumulated yet
    overflow |= mx > m_ref + kTauFixed;
  }
  const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float e = __builtin_amdgcn_exp2f(sacc[r] - m_use);
    psum += e;
    p[r >> 3][r & 7] = (_Float16)e;
  }
  l_sum += psum;
}

// Value product of one tile for this wave's 128 features and all 128 heads,
// with the staging of the next tile woven in.  MFMA I = 16 j + 4 f + hg
// accumulates O^T[feature block 4 wave + f][head group hg] over token half j.
// Each step holds one MFMA, the operand reads for four MFMAs later and one
// staging piece (an LDS store, or dequantisation and store for the quantised
// formats, followed by the load that refills the registers it freed), fenced so
// that the scheduler keeps that order: the staging work then executes in the
// shadow of the running MFMA, and the loads trickle out one per MFMA instead of
// stalling the wave on the address queue as a burst would.  P^T of
// token half j stays in pt[] while its 16 MFMAs run (the next half's fragment
// hg replaces it right after its last use); V^T fragments alternate between two
// buffers.
template <class Loader, class Begin>
struct H128Values {
  const char* buf;
  const char* pbuf;
  const H128Lane& L;
  int wave;
  floatx16 (&o)[16];
  Loader& ld;
  char* nxt;
  Begin& begin;
  half8 pt[4], vb[2];

  // V^T fragment (32 features x 16 tokens) for feature block 4 wave + f, token half j.
  __device__ __forceinline__ half8 vread(int j, int f) const {
    const int blk = 4 * wave + f;
    const uint32_t off = 16 * j * kRowLds + 128 * (blk >> 1);
    const half4 lo = lds_read_tr(buf, L.pv_off[blk & 1] + off);
    const half4 hi = lds_read_tr(buf, L.pv_off[2 + (blk & 1)] + off);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  __device__ __forceinline__ half8 pread(int j, int hg) const {
    return *reinterpret_cast<const half8*>(pbuf + hg * 32 * kPRow + L.p_off(j));
  }
  template <int I>
  __device__ __forceinline__ void step() {
    constexpr int j = I >> 4, f = (I >> 2) & 3, hg = I & 3;
    o[4 * f + hg] = mfma32x32x16(vb[f & 1], pt[hg], o[4 * f + hg]);
    if constexpr (hg == 0 && I + 4 < 32) vb[(f + 1) & 1] = vread((I + 4) >> 4, ((I + 4) >> 2) & 3);
    if constexpr (j == 0 && f == 3) pt[hg] = pread(1, hg);
    if constexpr (I < Loader::kStoreSteps) {
      ld.template store_step<I>(nxt);
      if constexpr (I == 0) begin();
      __builtin_amdgcn_sched_barrier(0);     // the refill may not overtake the store of the same registers
      ld.template load_step<I>();
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (I + 1 < 32) step<I + 1>();
  }
  __device__ __forceinline__ void run() {
    static_assert(Loader::kStoreSteps < 32, "staging must fit in the value product");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) pt[hg] = pread(0, hg);
    vb[0] = vread(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    step<0>();
  }
};

// The per-channel INT8 format splits a work item in two passes that share the
// softmax state: tokens of closed blocks [t_begin, closed_end), then the tile
// holding the open block, from open_begin (a multiple of the tile size kTile),
// tokens below open_lo masked (they were in the first pass).  closed_end is a
// multiple of 32 (or the item's end), so every 32 tokens of the first pass are
// all in range or all out.
struct Int8cSplit {
  int closed_end, open_begin, open_lo;
};
template <int kTile>
__device__ __forceinline__ Int8cSplit int8c_split(const DecodeArgs& a, const ItemRange& it) {
  const int ce = (a.seq_lens[it.b] / 32) * 32;   // end of the closed blocks
  Int8cSplit sp;
  sp.closed_end = min(it.t_end, max(it.t_begin, ce));
  sp.open_lo = max(it.t_begin, ce);
  sp.open_begin = sp.open_lo < it.t_end ? max(it.t_begin, ce & ~(kTile - 1)) : it.t_end;
  return sp;
}

// All store steps of a loader at once (when there is no value product to hide them in).
template <int I = 0, class Loader>
__device__ __forceinline__ void store_all(Loader& ld, char* buf) {
  if constexpr (I < Loader::kStoreSteps) {
    ld.template store_step<I>(buf);
    store_all<I + 1>(ld, buf);
  }
}

// One tile step: scores and softmax on `cur`, P exchange, then the value
// product with the next tile staged into `nxt`.  `cur` and `nxt` are distinct
// LDS arrays (the caller alternates them by unrolling), so the compiler can
// prove the staging writes never alias the operand reads and is free to
// interleave them.
template <class Loader, int kMode, class PageAt>
__device__ __forceinline__ void h128_step(const DecodeArgs& a, int s, int seg0, int seg1, const char* cur,
                                          char* nxt, char* pbuf, const char* qtail,
                                          const H128Lane& L, int wave,
                                          const half8 (&q)[kQReg], floatx16 (&o)[16], float& m_ref,
                                          float& l_sum, bool& overflow, Loader& ld, PageAt&& page_at) {
  __syncthreads();                         // tile s complete; P buffer and `nxt` free
  // Page ids of this tile and of the one staged after the next, read here, where no
  // other LDS access is in flight, and kept in SGPRs (a table read between the
  // value MFMAs would drain their operand reads).
  int pg0 = __builtin_amdgcn_readfirstlane((int)page_at(s));
  int pg2 = __builtin_amdgcn_readfirstlane((int)page_at(s + 2));
  asm volatile("" : "+s"(pg0), "+s"(pg2));
  const int t0 = seg0 + s * kTile128;
  half8 p[2];
  h128_scores<kMode, Loader::kScorePrefetch>(cur, qtail, L, q, m_ref, l_sum, overflow, t0, seg1, pg0 >= 0,
                                                  a.scale_log2, p);
  auto begin = [&]() { ld.begin(a, pg2, seg0 + (s + 2) * kTile128, seg1); };
  if (kMode != 1) {
    char* pw = pbuf + wave * 32 * kPRow;
    *reinterpret_cast<half8*>(pw + L.p_off(0)) = p[0];
    *reinterpret_cast<half8*>(pw + L.p_off(1)) = p[1];
    __syncthreads();                       // P of all heads visible
    H128Values<Loader, decltype(begin)>{cur, pbuf, L, wave, o, ld, nxt, begin}.run();
  } else {
    store_all(ld, nxt);
    ld.issue(a, pg2, seg0 + (s + 2) * kTile128, seg1);
  }
}

// Tokens [t_begin, t_end) of sequence b.  t_begin is a multiple of the page
// size, or the range fits one tile (the page table is sampled per 64 tokens
// from t_begin).
template <class Loader, int kMode>
__device__ __forceinline__ void h128_pass(const DecodeArgs& a, int b, int t_begin, int t_end, char* lds0, char* lds1,
                                          char* pbuf, const char* qtail, int32_t* ptab,
                                          const H128Lane& L,
                                          int wave, const half8 (&q)[kQReg], floatx16 (&o)[16], float& m_ref,
                                          float& l_sum, bool& overflow) {
  for (int seg0 = t_begin; seg0 < t_end; seg0 += kSegPages * kBlock) {
    const int seg1 = min(t_end, seg0 + kSegPages * kBlock);
    __syncthreads();                       // earlier users of the buffers and the table are done
    fill_ptab(a, b, seg0, seg1, ptab);
    __syncthreads();
    const int n_tiles = (seg1 - seg0 + kTile128 - 1) / kTile128;
    auto page_at = [&](int t) -> int64_t {       // -1 past the segment; branch free (read clamped, then select)
      const int pg = ptab[(min(t, n_tiles - 1) * kTile128) / kBlock];
      return t < n_tiles ? pg : -1;
    };
    Loader ld;
    ld.issue(a, page_at(0), seg0, seg1);
    ld.commit(lds0);
    ld.issue(a, page_at(1), seg0 + kTile128, seg1);
    for (int s = 0; s < n_tiles; s += 2) {
      h128_step<Loader, kMode>(a, s, seg0, seg1, lds0, lds1, pbuf, qtail, L, wave, q, o, m_ref, l_sum,
                               overflow, ld, page_at);
      if (s + 1 < n_tiles)
        h128_step<Loader, kMode>(a, s + 1, seg0, seg1, lds1, lds0, pbuf, qtail, L, wave, q, o, m_ref,
                                 l_sum, overflow, ld, page_at);
    }
  }
}

// One pass of the item in mode kMode: the format's loader over the whole range,
// or for the per-channel INT8 format its closed blocks and then its open block.
template <int kCache, int kMode>
__device__ __forceinline__ void h128_passes(const DecodeArgs& a, const ItemRange& it, char* lds0, char* lds1,
                                            char* pbuf, const char* qtail, int32_t* ptab, const H128Lane& L,
                                            int wave, const half8 (&q)[kQReg], floatx16 (&o)[16], float& m_ref,
                                            float& l_sum, bool& overflow) {
  if constexpr (kCache == 7) {
    const Int8cSplit sp = int8c_split<kTile128>(a, it);
    h128_pass<LoaderInt8cReg<kSwz128>, kMode>(a, it.b, it.t_begin, sp.closed_end, lds0, lds1, pbuf, qtail, ptab, L,
                                              wave, q, o, m_ref, l_sum, overflow);
    h128_pass<LoaderInt8cOpenReg<kSwz128>, kMode>(a, it.b, sp.open_begin, it.t_end, lds0, lds1, pbuf, qtail, ptab,
                                                  L, wave, q, o, m_ref, l_sum, overflow);
  } else {
    using Loader = typename std::conditional<
        kCache == 0, LoaderBf16Reg<kTile128, kSwz128>,
        typename std::conditional<kCache == 1 || kCache == 4 || kCache == 5,
                                  LoaderInt8Reg<kTile128, kSwz128, 0, kCache >= 4, kCache == 5>,
                                  LoaderInt4Reg<kTile128, kSwz128, 0, kCache == 3 || kCache == 6, kCache == 6>>::type>::type;
    h128_pass<Loader, kMode>(a, it.b, it.t_begin, it.t_end, lds0, lds1, pbuf, qtail, ptab, L, wave, q, o, m_ref,
                             l_sum, overflow);
  }
}

template <int kCache>
__global__ __launch_bounds__(256, 1) void decode_h128(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char lds0[kBuf128];
  __shared__ __attribute__((aligned(16))) char lds1[kBuf128];
  __shared__ __attribute__((aligned(16))) char pbuf[kPBuf];
  __shared__ __attribute__((aligned(16))) char qtail[kQTailBytes];
  __shared__ int32_t ptab[kSegPages];
  ItemRange it = item_range(a);
  if (!it.ok) return;
  if (a.num_pages <= 0) it.t_end = it.t_begin;     // no page can be valid (the loaders need page 0)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane & 31;
  const int g = lane >> 5;
  const int h = wave * 32 + hl;                    // this lane's head in the score phase
  const H128Lane L = h128_lane();

  // Q^T as the B operand: lane holds q_abs[b][h][16 ks + 8 g .. +7] for the
  // first kQReg k-steps; the rest of every head's row goes to LDS.
  half8 q[kQReg];
  {
    const uint16_t* qp = a.q_abs + ((int64_t)it.b * 128 + h) * kDk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kQReg; ++ks) q[ks] = __builtin_bit_cast(half8, ld16(qp + 16 * ks));
    const int hr = threadIdx.x >> 1, c0 = kQTail * (threadIdx.x & 1);
    const uint16_t* qr = a.q_abs + ((int64_t)it.b * 128 + hr) * kDk + 16 * kQReg;
#pragma unroll
    for (int c = c0; c < c0 + kQTail; ++c) *reinterpret_cast<u32x4*>(qtail + qtail_off(hr, c)) = ld16(qr + 8 * c);
  }
  // Retire the Q loads here: otherwise the compiler's wait for them sits inside
  // the tile loop and also drains the tile loads issued after them.
  wait_vm<0>();
  floatx16 o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = floatx16{};
  float m_ref = -INFINITY, l_sum = 0.f;
  bool overflow = false;

  h128_passes<kCache, 0>(a, it, lds0, lds1, pbuf, qtail, ptab, L, wave, q, o, m_ref, l_sum, overflow);
  if (__syncthreads_or(overflow)) {
    // Rare: some head's scores grew by more than 2^15 after its first tile.
    m_ref = -INFINITY;
    h128_passes<kCache, 1>(a, it, lds0, lds1, pbuf, qtail, ptab, L, wave, q, o, m_ref, l_sum, overflow);
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = floatx16{};
    l_sum = 0.f;
    h128_passes<kCache, 2>(a, it, lds0, lds1, pbuf, qtail, ptab, L, wave, q, o, m_ref, l_sum, overflow);
  }

  // ---- per-head sums from the owning waves, then normalise and write ----
  if constexpr (kCache == 2 || kCache == 3 || kCache == 6) {
    // INT4: o_part is stored straight from the accumulator layout (16-byte row
    // pieces): with the transposed write below, this kernel spills in its tile loop.
    const float l_tot = l_sum + __shfl_xor(l_sum, 32, 64);
    float* red = reinterpret_cast<float*>(pbuf);
    __syncthreads();                                 // every wave is done with the P buffer
    if (g == 0) red[h] = l_tot;
    __syncthreads();
    float inv[4];
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
      const float l = red[32 * hg + hl];
      inv[hg] = l > 0.f ? 1.f / l : 0.f;
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
#pragma unroll
      for (int hg = 0; hg < 4; ++hg) {
        uint16_t* op = a.o_part + ((int64_t)it.out_row * 128 + 32 * hg + hl) * kDc + 128 * wave + 32 * f + 4 * g;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const floatx16& v = o[4 * f + hg];
          const floatx4 x = floatx4{v[4 * rr], v[4 * rr + 1], v[4 * rr + 2], v[4 * rr + 3]} * inv[hg];
          *reinterpret_cast<half4*>(op + 8 * rr) = __builtin_convertvector(x, half4);   // round to nearest even
        }
      }
    }
    if (g == 0) a.lse_part[(int64_t)it.out_row * 128 + h] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    // Lane indices are recomputed here from an opaque copy of the thread id, so
    // that no epilogue offset is kept live (in VGPRs) across the tile loop.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int elane = tid & 63, ehl = elane & 31, eg = elane >> 5, eh = wave * 32 + ehl;
    const float l_tot = l_sum + __shfl_xor(l_sum, 32, 64);
    float* red = reinterpret_cast<float*>(pbuf);
    __syncthreads();                                 // every wave is done with the P buffer
    if (eg == 0) red[eh] = l_tot;
    __syncthreads();
    float inv[4];
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
      const float l = red[32 * hg + ehl];
      inv[hg] = l > 0.f ? 1.f / l : 0.f;
    }
    // o_part rows leave through LDS so that every store writes whole 256-byte row
    // pieces (16 lanes per row) instead of 16-byte fragments of 32 rows.  Each wave
    // transposes its own features [128 wave, +128) of 64 heads at a time in a
    // private 16 KB region (rows of 256 B, 16-byte chunk c at c ^ (row & 15)).
    char* xbuf = (wave < 2 ? lds0 : lds1) + (wave & 1) * 16384;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int hgi = 0; hgi < 2; ++hgi) {
        const int hg = 2 * hh + hgi, row = 32 * hgi + ehl;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            // features 32 f + 16 pr + 8 j + 4 eg + 0..3 of this lane's head (j = 0, 1)
            const floatx16& v = o[4 * f + hg];
            u32x2 x[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int r0 = 4 * (2 * pr + j);
              const floatx4 y = floatx4{v[r0], v[r0 + 1], v[r0 + 2], v[r0 + 3]} * inv[hg];
              x[j] = __builtin_bit_cast(u32x2, __builtin_convertvector(y, half4));   // round to nearest even
            }
            // v_permlane32_swap exchanges the upper half-wave of its first operand with
            // the lower half-wave of its second: afterwards the lane of half eg holds the eight
            // consecutive features 8 (1 - eg) .. +7 of this 16-feature pair as (x[1], x[0]).
#pragma unroll
            for (int d = 0; d < 2; ++d) {
              const auto sw = __builtin_amdgcn_permlane32_swap(x[1][d], x[0][d], false, false);
              x[1][d] = sw[0];
              x[0][d] = sw[1];
            }
            const int chunk = 4 * f + 2 * pr + 1 - eg;
            *reinterpret_cast<u32x4*>(xbuf + row * 256 + 16 * (chunk ^ (row & 15))) =
                u32x4{x[1][0], x[1][1], x[0][0], x[0][1]};
          }
        }
      }
      asm volatile("" ::: "memory");           // this wave's LDS writes before its reads (in-order per wave)
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int row = 4 * k + (elane >> 4), chunk = elane & 15;
        const u32x4 v = *reinterpret_cast<const u32x4*>(xbuf + row * 256 + 16 * (chunk ^ (row & 15)));
        st16(a.o_part + ((int64_t)it.out_row * 128 + 64 * hh + row) * kDc + 128 * wave + 8 * chunk, v);
      }
      asm volatile("" ::: "memory");           // reads done before the next half overwrites the region
    }
    if (eg == 0) a.lse_part[(int64_t)it.out_row * 128 + eh] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ===========================================================================
// H = 16
// ===========================================================================
constexpr int kTile16 = 64;
constexpr int kBuf16 = kTile16 * kRowLds;          // 73,728 B
// Q^T of the first kQ16Reg k-steps (32 columns each) stays in VGPRs; the other
// k-steps sit in LDS as the register image of a wave (k-step j: 64 lanes x 16 B,
// lane l at 16 l), which leaves the VGPRs for two staged tiles.
constexpr int kQ16Reg = 10, kQ16Lds = kDk / 32 - kQ16Reg;

// The work-group has 8 waves.  Waves 0-3 compute: wave w takes tokens 16 w ..
// 16 w + 15 of each 64-token tile for all 16 heads (mfma 16x16x32 scores,
// 16x16x16 values); their (max, sum, O) are merged through LDS at the end.
// Waves 4-7 only stage tiles: they hold the next two tiles in VGPRs, write tile
// s + 1 (widened or dequantised to fp16) into the free LDS buffer while the
// compute waves work on tile s, and then issue the loads of tile s + 3.  Each
// SIMD runs one wave of each kind and interleaves them, so the staging work and
// the compute overlap, and every tile's loads have two tile steps to arrive.
// A staging step's store of one tile and load of the next: interleaved by the
// loader when it provides commit_issue, else one after the other.
template <class L>
__device__ __forceinline__ auto stage_commit_issue(L& ld, char* buf, const DecodeArgs& a, int64_t page, int t0,
                                                   int t_end, int) -> decltype(ld.commit_issue(buf, a, page, t0, t_end)) {
  return ld.commit_issue(buf, a, page, t0, t_end);
}
template <class L>
__device__ __forceinline__ void stage_commit_issue(L& ld, char* buf, const DecodeArgs& a, int64_t page, int t0,
                                                   int t_end, long) {
  ld.commit(buf);
  ld.issue(a, page, t0, t_end);
}

// Staging waves of decode_h16: the same segment loop and barriers as the compute
// waves.  Stage (s + 1) % 2 holds tile s + 1 (written at step s, then reloaded
// with tile s + 3); the other holds tile s + 2.
template <class Loader>
__device__ __forceinline__ void h16_stage(const DecodeArgs& a, int b, int t_begin, int t_end, int t_lo, char* lds,
                                          int32_t* ptab, bool filled = false) {
  for (int seg0 = t_begin; seg0 < t_end; seg0 += kSegPages * kBlock) {
    const int seg1 = min(t_end, seg0 + kSegPages * kBlock);
    __syncthreads();                       // earlier users of the buffers and the table are done
    if (!(filled && seg0 == t_begin)) fill_ptab(a, b, seg0, seg1, ptab);
    __syncthreads();
    const int n_tiles = (seg1 - seg0 + kTile16 - 1) / kTile16;
    // Every step commits and issues unconditionally (tiles past the end load
    // the zero page and land in the idle buffer).  The loads are the loaders'
    // tied assembly loads, so the waits are explicit: a commit waits until only
    // the other loader's tile is in flight.
    Loader ld0, ld1;
    ld0.set_lo(t_lo);
    ld1.set_lo(t_lo);
    ld0.issue(a, ptab[0], seg0, seg1);
    ld1.issue(a, n_tiles > 1 ? ptab[1] : -1, seg0 + kTile16, seg1);
    wait_vm<Loader::kLoads>();             // tile 0; tile 1 stays in flight
    ld0.settle_all();
    ld0.commit(lds);
    ld0.issue(a, n_tiles > 2 ? ptab[2] : -1, seg0 + 2 * kTile16, seg1);
    auto stage_step = [&](int s, Loader& ldn) {
      __syncthreads();
      // The page id is read before the tile's LDS stores are issued, so that
      // waiting for it does not wait for them to drain.
      const int next_page = s + 3 < n_tiles ? ptab[s + 3] : -1;
      wait_vm<Loader::kLoads>();           // the other loader's tile stays in flight
      ldn.settle_all();
      stage_commit_issue(ldn, lds + ((s + 1) & 1) * kBuf16, a, next_page, seg0 + (s + 3) * kTile16, seg1, 0);
    };
    // Pairs of steps (an odd tile count gets one idle step, matched by an extra
    // barrier in the compute waves).
    for (int s = 0; s < n_tiles; s += 2) {
      stage_step(s, ld1);
      stage_step(s + 1, ld0);
    }
    wait_vm<0>();                          // the last (zero-page) tiles
  }
}

// OpenLoader (not void): the two-pass form above, Loader taking the closed blocks.
template <class Loader, class OpenLoader = void>
__global__ __launch_bounds__(512, 1) void decode_h16(DecodeArgs a) {
  constexpr bool kSplit = !std::is_same<OpenLoader, void>::value;
  __shared__ __attribute__((aligned(16))) char lds[2 * kBuf16];
  __shared__ __attribute__((aligned(16))) char qt16[kQ16Lds * 1024];
  __shared__ int32_t ptab[kSegPages];
  ItemRange it = item_range(a);
  if (!it.ok) return;
  if (a.num_pages <= 0) it.t_end = it.t_begin;     // no page can be valid (the loaders need page 0)
  const bool stager = threadIdx.x >= 256;          // waves 4-7 (uniform per wave)
  const int lane = threadIdx.x & 63;
  const int wave = (threadIdx.x >> 6) & 3;
  const int hl = lane & 15;          // head (MFMA column)
  const int grp = lane >> 4;         // 0..3

  // Q^T k-steps past kQ16Reg go to LDS (all threads), the rest to the compute
  // waves' VGPRs below.
  // With one pass, the page table of its first segment is requested together
  // with the Q^T tail (one memory round trip instead of two); that segment then
  // skips its fill.
  static_assert(kQ16Lds * 64 == 512 && kSegPages <= 2 * 512, "one Q^T chunk and two table entries per thread");
  {
    const int l = threadIdx.x & 63;
    const u32x4 qv = ld16(a.q_abs + ((int64_t)it.b * 16 + (l & 15)) * kDk + 32 * (kQ16Reg + (threadIdx.x >> 6)) +
                          8 * (l >> 4));
    if constexpr (!kSplit) {
      const int seg1 = it.t_begin + min(it.t_end - it.t_begin, kSegPages * kBlock);
      const int n0 = (seg1 - it.t_begin + kBlock - 1) / kBlock;
      const int i0 = threadIdx.x, i1 = threadIdx.x + 512;
      const int32_t p0 = i0 < n0 ? (int32_t)page_of(a, it.b, it.t_begin + i0 * kBlock) : -1;
      const int32_t p1 = i1 < n0 ? (int32_t)page_of(a, it.b, it.t_begin + i1 * kBlock) : -1;
      *reinterpret_cast<u32x4*>(qt16 + 16 * threadIdx.x) = qv;
      if (i0 < n0) ptab[i0] = p0;
      if (i1 < n0) ptab[i1] = p1;
    } else {
      *reinterpret_cast<u32x4*>(qt16 + 16 * threadIdx.x) = qv;
    }
  }
  if (stager) {
    wait_vm<0>();
    if constexpr (kSplit) {
      const Int8cSplit sp = int8c_split<kTile16>(a, it);
      h16_stage<Loader>(a, it.b, it.t_begin, sp.closed_end, it.t_begin, lds, ptab);
      h16_stage<OpenLoader>(a, it.b, sp.open_begin, it.t_end, sp.open_lo, lds, ptab);
    } else {
      h16_stage<Loader>(a, it.b, it.t_begin, it.t_end, it.t_begin, lds, ptab, true);
    }
    __syncthreads();                       // the two barriers of the compute waves' merge
    __syncthreads();
    return;
  }
  // Q^T as the B operand of 16x16x32: lane holds q_abs[b][hl][32 ks + 8 grp .. +7].
  half8 q[kQ16Reg];
  {
    const uint16_t* qp = a.q_abs + ((int64_t)it.b * 16 + hl) * kDk + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < kQ16Reg; ++ks) q[ks] = __builtin_bit_cast(half8, ld16(qp + 32 * ks));
  }
  // Retire the Q loads here: otherwise the compiler's wait for them sits inside
  // the tile loop and also drains the tile loads.
  wait_vm<0>();
  floatx4 o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = floatx4{};
  float m_run = -INFINITY;
  float l_sum = 0.f;

  // Score operand: row tw + hl, chunk 4 ks + grp.  Transposed value read:
  // row tw + 4 grp + (hl >> 2), chunk 2 tile + ((hl & 3) >> 1), +8 B when hl odd.
  const int tw = 16 * wave;                                          // this wave's rows
  uint32_t qk_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) qk_off[par] = swz<kSwz16>(tw + hl, 4 * par + grp);
  const int pv_row = tw + 4 * grp + (hl >> 2);
  uint32_t pv_off[4];
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4) pv_off[t4] = swz<kSwz16>(pv_row, 2 * t4 + ((hl & 3) >> 1)) + 8 * (hl & 1);

  // Tokens [t_begin, t_end) of the item; rows below t_lo are masked.
  auto pass = [&](int t_begin, int t_end, int t_lo, bool filled) {
  for (int seg0 = t_begin; seg0 < t_end; seg0 += kSegPages * kBlock) {
    const int seg1 = min(t_end, seg0 + kSegPages * kBlock);
    __syncthreads();                       // earlier users of the buffers and the table are done
    if (!(filled && seg0 == t_begin)) fill_ptab(a, it.b, seg0, seg1, ptab);
    __syncthreads();
    const int n_tiles = (seg1 - seg0 + kTile16 - 1) / kTile16;
    // One barrier per tile, as in h16_stage: at the barrier of step s, tile s is
    // complete in buffer s % 2 and buffer (s + 1) % 2 is free.
    for (int s = 0; s < n_tiles; ++s) {
      __syncthreads();
      const char* buf = lds + (s & 1) * kBuf16;
      const int t0 = seg0 + s * kTile16;
      const bool page_ok = ptab[s] >= 0;

      // Scores: 18 k-steps as two interleaved chains, the K (and, past kQ16Reg,
      // Q^T) fragments read kPf steps ahead, one fenced step per MFMA.
      constexpr int kSteps = kDk / 32, kPf = 4;
      __builtin_amdgcn_sched_barrier(0);
      floatx4 sacc0 = floatx4{}, sacc1 = floatx4{};
      half8 kb[kPf], qb[kPf];
      auto kread = [&](int ks) { return *reinterpret_cast<const half8*>(buf + qk_off[ks & 1] + 128 * (ks >> 1)); };
      auto qread = [&](int ks) { return *reinterpret_cast<const half8*>(qt16 + (ks - kQ16Reg) * 1024 + 16 * lane); };
#pragma unroll
      for (int d = 0; d < kPf; ++d) kb[d] = kread(d);
      static_assert(kQ16Reg >= kPf, "the first Q^T fragments come from VGPRs");
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks) {
        const half8 qv = ks < kQ16Reg ? q[ks < kQ16Reg ? ks : 0] : qb[ks % kPf];
        if (ks & 1) sacc1 = mfma16x16x32(kb[ks % kPf], qv, sacc1);
        else sacc0 = mfma16x16x32(kb[ks % kPf], qv, sacc0);
        const int kn = ks + kPf;
        if (kn < kSteps) {
          kb[ks % kPf] = kread(kn);
          if (kn >= kQ16Reg) qb[ks % kPf] = qread(kn);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      floatx4 sacc = sacc0 + sacc1;
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tt = t0 + tw + 4 * grp + r;
        float v = sacc[r] * a.scale_log2;
        if (!page_ok || tt >= seg1 || (kSplit && tt < t_lo)) v = -INFINITY;
        sacc[r] = v;
        mx = fmaxf(mx, v);
      }
      mx = max_xor16_32(mx);
      const bool need = mx > m_run + kTau;
      if (__ballot(need)) {
        const float m_new = need ? mx : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) o[i] *= alpha;
        l_sum *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      half4 p;
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __builtin_amdgcn_exp2f(sacc[r] - m_use);
        psum += e;
        p[r] = (_Float16)e;
      }
      l_sum += psum;
#pragma unroll
      for (int tile = 0; tile < 32; ++tile) {
        const half4 av = lds_read_tr(buf, pv_off[tile & 3] + 128 * (tile >> 2));
        o[tile] = mfma16x16x16(av, p, o[tile]);
      }
    }
    if (n_tiles & 1) __syncthreads();      // the staging waves' idle step
  }
  };
  if constexpr (kSplit) {
    const Int8cSplit sp = int8c_split<kTile16>(a, it);
    pass(it.t_begin, sp.closed_end, it.t_begin, false);
    pass(sp.open_begin, it.t_end, sp.open_lo, false);
  } else {
    pass(it.t_begin, it.t_end, it.t_begin, true);
  }

  // ---- merge the four waves (each saw a quarter of every page) ----
  float l_w = l_sum;
  l_w += __shfl_xor(l_w, 16, 64);
  l_w += __shfl_xor(l_w, 32, 64);
  __syncthreads();                                   // all waves done with the tiles
  // [4 waves][16 heads] rows of O padded to kRed floats (the 16-byte pad puts
  // the 16 heads a store instruction writes on distinct banks), then [4][16] m,
  // [4][16] l.
  constexpr int kRed = kDc + 4;
  static_assert((4 * 16 * kRed + 128) * 4 <= 2 * kBuf16, "the merge fits in the tile buffers");
  float* red = reinterpret_cast<float*>(lds);
  float* red_m = red + 4 * 16 * kRed;
  float* red_l = red_m + 64;
  {
#pragma unroll
    for (int tile = 0; tile < 32; ++tile)       // features 16 tile + 4 grp .. +3 of head hl
      *reinterpret_cast<floatx4*>(red + (wave * 16 + hl) * kRed + 16 * tile + 4 * grp) = o[tile];
    if (grp == 0) {
      red_m[wave * 16 + hl] = m_run;
      red_l[wave * 16 + hl] = l_w;
    }
  }
  __syncthreads();
  {
    // 16 threads per head; thread i takes features 4 i + 64 j .. +3 (j < 8), so
    // that each read and store instruction covers contiguous bytes of four rows.
    const int head = threadIdx.x >> 4;               // 0..15
    const int ci = threadIdx.x & 15;
    float mw[4], m = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) { mw[w] = red_m[w * 16 + head]; m = fmaxf(m, mw[w]); }
    float ew[4], l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      ew[w] = (mw[w] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw[w] - m);
      l += ew[w] * red_l[w * 16 + head];
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* op = a.o_part + ((int64_t)it.out_row * 16 + head) * kDc;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int f = 4 * ci + 64 * j;
      floatx4 v = floatx4{};
#pragma unroll
      for (int w = 0; w < 4; ++w) v += ew[w] * *reinterpret_cast<const floatx4*>(red + (w * 16 + head) * kRed + f);
      *reinterpret_cast<half4*>(op + f) = __builtin_convertvector(v * inv, half4);   // nearest even
    }
    if ((threadIdx.x & 15) == 0)
      a.lse_part[(int64_t)it.out_row * 16 + head] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// ===========================================================================
// H = 16, FP8 (e4m3, per-token scale) cache on the FP8 matrix instructions
// ===========================================================================
// Both products run on v_mfma_scale_f32_16x16x128_f8f6f4 with the cache's own
// e4m3 codes as one operand, so the staging waves copy raw page bytes into LDS
// and dequantise nothing:
//   scores  S^T[tokens][heads] = K[tokens][128 ch] . q~^T, four K-steps over the
//           512 latent channels.  q~ goes in as two e4m3 terms with a power-of-
//           two scale per head (hi = e4m3(q~ 2^-e), lo = e4m3((q~ 2^-e - hi) 2^4)),
//           both terms into one accumulator through the instruction's block
//           scales (2^e and 2^(e-4)); the token's fp32 scale multiplies the
//           result row.  The RoPE key (per-8-group scales) is widened to fp16 in
//           registers for two 16x16x32 fp16 products.
//   values  O^T[features][heads] += V^T[features][128 tokens] . P'', with
//           P' = P * (token scale) and P'' its two e4m3 terms under a power-of-
//           two scale per 32-token block and head, passed as the block scales of
//           the B operand; V^T comes from the raw tile by 8-bit transposed LDS
//           reads (ds_read_b64_tr_b8).
// The two-term split keeps each operand to about 2^-8 relative (the precision
// contract's FP8 case); two FP8 products take the matrix core as long as one
// fp16 product of the same shape, so what this gains is staging work and LDS
// bytes, and with them a second 128-token tile in flight per CU.
//
// Instruction layout (16x16x128, 8-bit operands; established by in-bounds
// probes on gfx950): lane l = 16 g + r holds row (or column) r; its byte j is
// K = 64 (j / 16) + 16 g + j % 16; the block scale of K-block b (K 32 b .. +31)
// of row r is the scale operand of lane 16 b + r; the result lane l holds rows
// 4 g .. 4 g + 3 of column r.
//
// Work-group: waves 0-3 compute, waves 4-7 stage (as decode_h16).  128-token
// tiles (two pages); compute wave w takes the scores of tokens 32 w .. 32 w + 31
// (K-block w of the value product) and the value product of features
// 128 w .. 128 w + 127 for all 16 heads, so the softmax maximum and P cross the
// waves through LDS (three barriers per tile) and no merge is needed at the end.
typedef int int32x8 __attribute__((ext_vector_type(8)));
typedef int int32x2 __attribute__((ext_vector_type(2)));

constexpr int kTileF8 = 128;
constexpr int kRowF8 = 576;                               // raw row: 512 latent codes, 64 RoPE-key codes
constexpr int kPageF8 = kBlock * 612;                     // [64][576] codes | [64] f32 | [64][8] f32
constexpr int kPgLatScale = 64 * 576, kPgKeyScale = kPgLatScale + 64 * 4;
constexpr int kF8LatScale = kTileF8 * kRowF8;             // LDS tile: rows | [128] f32 | [128][8] f32
constexpr int kF8KeyScale = kF8LatScale + kTileF8 * 4;
constexpr int kBufF8 = kF8KeyScale + kTileF8 * 32;        // 78,336 B
constexpr int kPexF8 = 2 * 16 * kTileF8;                  // P'' terms: [2][16 heads][128 tokens] bytes
constexpr int kSegPagesF8 = 256;

// Raw-row swizzle: 16-byte chunk c of row r sits at chunk c ^ f8_swz(r) (low two
// bits), so that the score reads (16 consecutive rows, one chunk) and the
// transposed reads (rows 16 g + j and 16 g + 16 + j for the two lane groups of
// a pass, or their +64 copies) hit 16 different bank quads.
__device__ __forceinline__ uint32_t f8_swz(int r) { return ((r >> 2) & 1) | ((((r >> 3) ^ (r >> 4)) & 1) << 1); }
__device__ __forceinline__ uint32_t f8_off(int r, int c) { return r * kRowF8 + 16 * (c ^ f8_swz(r)); }
// P'' exchange: head h's 128 bytes of term t, 16-byte chunk c at c ^ ((h >> 1) & 7).
__device__ __forceinline__ uint32_t pex_off(int t, int h, int c) { return t * 2048 + h * 128 + 16 * (c ^ ((h >> 1) & 7)); }

__device__ __forceinline__ floatx4 mfma_f8(int32x8 a, int32x8 b, floatx4 c, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}
// Power-of-two exponent that maps a positive maximum m into [128, 256): m 2^-e,
// clamped to [-120, 120] so that the block scales 127 + e and 127 + e - 4 stay
// valid E8M0 codes (a smaller maximum, e.g. subnormal, only lets its block's
// values underflow: they are below 2^-113 of the largest).
__device__ __forceinline__ int f8_exp(float m) {
  const int e = m > 0.f ? (int)((__float_as_uint(m) >> 23) & 0xffu) - 127 - 7 : 0;
  return min(max(e, -120), 120);
}
// Two e4m3 terms of v (|v| < 256): hi = e4m3(v), lo = e4m3((v - hi) 2^4), packed
// four values per word.
__device__ __forceinline__ void f8_split4(const float (&v)[4], uint32_t& hi, uint32_t& lo) {
  uint32_t h = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
  h = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], (int)h, true);
  float r[4];
  r[0] = (v[0] - __builtin_amdgcn_cvt_f32_fp8((int)h, 0)) * 16.f;
  r[1] = (v[1] - __builtin_amdgcn_cvt_f32_fp8((int)h, 1)) * 16.f;
  r[2] = (v[2] - __builtin_amdgcn_cvt_f32_fp8((int)h, 2)) * 16.f;
  r[3] = (v[3] - __builtin_amdgcn_cvt_f32_fp8((int)h, 3)) * 16.f;
  uint32_t l = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
  l = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], (int)l, true);
  hi = h;
  lo = l;
}

// Staging of one raw 128-token tile (threads kTid0 .. kTid0 + 255).  Load i of
// thread t is 16-byte chunk t + 256 (i % 9) of page i / 9's code block (2,304
// chunks: row = chunk / 36, column chunk % 36), so that consecutive lanes read
// consecutive bytes; plus 16 bytes of the key scales and 16 bytes of the latent
// scales (stored by t < 32 only; every thread loads, so that each wave issues
// the same number of loads).  Rows past t_end and pages out of range read the
// zero page.
template <int kTid0>
struct LoaderF8Raw {
  static constexpr int kLoads = 20;
  u32x4 c[18] = {};
  u32x4 ks = {}, ls = {};

  template <int I>
  __device__ __forceinline__ void issue_one(const DecodeArgs& a, int64_t pgi, int t0, int t_end) {
    const int q = ltid<kTid0>() + 256 * (I % 9), row = q / 36;
    const uint8_t* src = page_base(a, pgi, pgi >= 0 && t0 + 64 * (I / 9) + row < t_end, kPageF8) + 16 * q;
    asm_ld16_nt<0>(c[I], src);
  }
  __device__ __forceinline__ void issue(const DecodeArgs& a, int64_t p0, int64_t p1, int t0, int t_end) {
    issue_one<0>(a, p0, t0, t_end);
    issue_one<1>(a, p0, t0, t_end);
    issue_one<2>(a, p0, t0, t_end);
    issue_one<3>(a, p0, t0, t_end);
    issue_one<4>(a, p0, t0, t_end);
    issue_one<5>(a, p0, t0, t_end);
    issue_one<6>(a, p0, t0, t_end);
    issue_one<7>(a, p0, t0, t_end);
    issue_one<8>(a, p0, t0, t_end);
    issue_one<9>(a, p1, t0, t_end);
    issue_one<10>(a, p1, t0, t_end);
    issue_one<11>(a, p1, t0, t_end);
    issue_one<12>(a, p1, t0, t_end);
    issue_one<13>(a, p1, t0, t_end);
    issue_one<14>(a, p1, t0, t_end);
    issue_one<15>(a, p1, t0, t_end);
    issue_one<16>(a, p1, t0, t_end);
    issue_one<17>(a, p1, t0, t_end);
    const int t = ltid<kTid0>();
    const int64_t pk = t < 128 ? p0 : p1;
    asm_ld16_nt<0>(ks, page_base(a, pk, pk >= 0, kPageF8) + kPgKeyScale + 16 * (t & 127));
    const int64_t pl = (t & 31) < 16 ? p0 : p1;
    asm_ld16_nt<0>(ls, page_base(a, pl, pl >= 0, kPageF8) + kPgLatScale + 16 * (t & 15));
  }
  __device__ __forceinline__ void settle_all() {
#pragma unroll
    for (int i = 0; i < 18; ++i) settle(c[i]);
    settle(ks);
    settle(ls);
  }
  __device__ __forceinline__ void commit(char* buf) {
    const int t = ltid<kTid0>();
#pragma unroll
    for (int i = 0; i < 18; ++i) {
      const int q = t + 256 * (i % 9), row = q / 36;
      *reinterpret_cast<u32x4*>(buf + f8_off(64 * (i / 9) + row, q - 36 * row)) = c[i];
    }
    *reinterpret_cast<u32x4*>(buf + kF8KeyScale + 2048 * (t >> 7) + 16 * (t & 127)) = ks;
    if (t < 32) *reinterpret_cast<u32x4*>(buf + kF8LatScale + 256 * (t >> 4) + 16 * (t & 15)) = ls;
  }
};

__device__ __forceinline__ void fill_ptab_n(const DecodeArgs& a, int b, int t0, int t1, int32_t* ptab) {
  const int n = (t1 - t0 + kBlock - 1) / kBlock;
  for (int i = threadIdx.x; i < n; i += blockDim.x) ptab[i] = (int32_t)page_of(a, b, t0 + i * kBlock);
}

__global__ __launch_bounds__(512, 1) void decode_h16f8(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kBufF8];
  __shared__ __attribute__((aligned(16))) char pex[kPexF8];
  __shared__ float xmax[4][16];            // per wave and head: the tile maximum, then (end) the sum
  __shared__ int xexp[4][16];              // per 32-token block and head: P'' exponent
  __shared__ int32_t ptab[kSegPagesF8];
  ItemRange it = item_range(a);
  if (!it.ok) return;
  if (a.num_pages <= 0) it.t_end = it.t_begin;     // no page can be valid (the loaders need page 0)
  const bool stager = threadIdx.x >= 256;          // waves 4-7 (uniform per wave)
  const int lane = threadIdx.x & 63;
  const int w = (threadIdx.x >> 6) & 3;
  const int r = lane & 15, g = lane >> 4;          // MFMA row/column r, lane group g

  if (stager) {
    for (int seg0 = it.t_begin; seg0 < it.t_end; seg0 += kSegPagesF8 * kBlock) {
      const int seg1 = min(it.t_end, seg0 + kSegPagesF8 * kBlock);
      __syncthreads();                     // earlier users of the buffers and the table are done
      fill_ptab_n(a, it.b, seg0, seg1, ptab);
      __syncthreads();
      const int n_tiles = (seg1 - seg0 + kTileF8 - 1) / kTileF8;
      const int n_pg = (seg1 - seg0 + kBlock - 1) / kBlock;
      auto pg = [&](int i) -> int64_t { return i < n_pg ? ptab[i] : -1; };
      LoaderF8Raw<256> ld0, ld1;
      ld0.issue(a, pg(0), pg(1), seg0, seg1);
      wait_vm<0>();
      ld0.settle_all();
      ld0.commit(lds);
      ld1.issue(a, pg(2), pg(3), seg0 + kTileF8, seg1);
      ld0.issue(a, pg(4), pg(5), seg0 + 2 * kTileF8, seg1);
      auto stage_step = [&](int s, LoaderF8Raw<256>& ldn) {
        __syncthreads();                   // X1: tile s in place, buffer (s + 1) % 2 free
        const int64_t q0 = pg(2 * s + 6), q1 = pg(2 * s + 7);
        wait_vm<LoaderF8Raw<256>::kLoads>();   // the other loader's tile stays in flight
        ldn.settle_all();
        ldn.commit(lds + ((s + 1) & 1) * kBufF8);
        ldn.issue(a, q0, q1, seg0 + (s + 3) * kTileF8, seg1);
        __syncthreads();                   // X2 (the compute waves' maximum exchange)
        __syncthreads();                   // X3 (their P exchange)
      };
      for (int s = 0; s < n_tiles; s += 2) {
        stage_step(s, ld1);
        stage_step(s + 1, ld0);
      }
      wait_vm<0>();                        // the last (zero-page) tiles
    }
    __syncthreads();                       // the compute waves' final sum exchange
    return;
  }

  // ---- compute waves: q~ as two e4m3 terms (lane: head r, channels of K-step s
  // 128 s + 16 g + 0..15 and 128 s + 64 + 16 g + 0..15), the RoPE part in fp16
  // (16x16x32 B operand: channels 512 + 8 g + 32 j .. +7).
  int32x8 qh[4], ql[4];
  half8 qr[2];
  int eq;                                  // per-head exponent of q~
  {
    const uint16_t* qp = a.q_abs + ((int64_t)it.b * 16 + r) * kDk;
    half8 x[4][4];                         // K-step s, piece 2 hh + k: channels 128 s + 64 hh + 16 g + 8 k .. +7
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int k = 0; k < 4; ++k) x[s][k] = __builtin_bit_cast(half8, ld16(qp + 128 * s + 64 * (k >> 1) + 16 * g + 8 * (k & 1)));
#pragma unroll
    for (int j = 0; j < 2; ++j) qr[j] = __builtin_bit_cast(half8, ld16(qp + kDc + 8 * g + 32 * j));
    float m = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)x[s][k][e]));
    m = wave_max_xor(m, 16);
    m = wave_max_xor(m, 32);                // all 512 channels of head r
    eq = f8_exp(m);
    const float sc = __uint_as_float((uint32_t)(127 - eq) << 23);   // 2^-eq
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const half8& xs = x[s][d >> 1];
        const int e0 = 4 * (d & 1);
        const float x4[4] = {(float)xs[e0] * sc, (float)xs[e0 + 1] * sc, (float)xs[e0 + 2] * sc, (float)xs[e0 + 3] * sc};
        uint32_t hi, lo;
        f8_split4(x4, hi, lo);
        qh[s][d] = (int)hi;
        ql[s][d] = (int)lo;
      }
  }
  wait_vm<0>();
  const int sq_hi = 127 + eq, sq_lo = 127 + eq - 4;
  floatx4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = floatx4{};
  float m_run = -INFINITY, l_sum = 0.f;

  for (int seg0 = it.t_begin; seg0 < it.t_end; seg0 += kSegPagesF8 * kBlock) {
    const int seg1 = min(it.t_end, seg0 + kSegPagesF8 * kBlock);
    __syncthreads();
    fill_ptab_n(a, it.b, seg0, seg1, ptab);
    __syncthreads();
    const int n_tiles = (seg1 - seg0 + kTileF8 - 1) / kTileF8;
    const int n_pg = (seg1 - seg0 + kBlock - 1) / kBlock;
    for (int s = 0; s < n_tiles; ++s) {
      __syncthreads();                     // X1
      const char* buf = lds + (s & 1) * kBufF8;
      const int t0 = seg0 + s * kTileF8;
      // ---- scores of tokens 32 w + 16 rb + 0..15 (rows), all heads (columns)
      float p[2][4];
      float lat[2][4];
      float mx = -INFINITY;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int row = 32 * w + 16 * rb + r;
        floatx4 acc = floatx4{}, accr = floatx4{};
        auto kread = [&](int s4) {
          const u32x4 k0 = *reinterpret_cast<const u32x4*>(buf + f8_off(row, 8 * s4 + g));
          const u32x4 k1 = *reinterpret_cast<const u32x4*>(buf + f8_off(row, 8 * s4 + 4 + g));
          return int32x8{(int)k0[0], (int)k0[1], (int)k0[2], (int)k0[3], (int)k1[0], (int)k1[1], (int)k1[2], (int)k1[3]};
        };
        int32x8 ka = kread(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          int32x8 kn = ka;
          if (s4 + 1 < 4) kn = kread(s4 + 1);
          acc = mfma_f8(ka, qh[s4], acc, 127, sq_hi);
          acc = mfma_f8(ka, ql[s4], acc, 127, sq_lo);
          ka = kn;
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // RoPE key codes 8 g + 32 j .. +7 of the row (chunk 32 + 2 j + g / 2, half g % 2) and their group scale
          const u32x2 kc = *reinterpret_cast<const u32x2*>(buf + f8_off(row, 32 + 2 * j + (g >> 1)) + 8 * (g & 1));
          const float ksc = reinterpret_cast<const float*>(buf + kF8KeyScale)[row * 8 + g + 4 * j];
          const _Float16 s256 = (_Float16)(ksc * 256.f);
          const u32x2 lo = fp8x4_to_f16(kc[0], half2v{s256, s256}), hi = fp8x4_to_f16(kc[1], half2v{s256, s256});
          const half8 kr = __builtin_bit_cast(half8, u32x4{lo[0], lo[1], hi[0], hi[1]});
          accr = mfma16x16x32(kr, qr[j], accr);
        }
        // result rows 32 w + 16 rb + 4 g + i
        const floatx4 ls = *reinterpret_cast<const floatx4*>(buf + kF8LatScale + 4 * (32 * w + 16 * rb + 4 * g));
        const bool page_ok = (2 * s + ((32 * w + 16 * rb) >> 6) < n_pg) &&
                             ptab[min(2 * s + ((32 * w + 16 * rb) >> 6), n_pg - 1)] >= 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tt = t0 + 32 * w + 16 * rb + 4 * g + i;
          const bool ok = page_ok && tt < seg1;
          float v = (acc[i] * ls[i] + accr[i]) * a.scale_log2;
          v = ok ? v : -INFINITY;
          p[rb][i] = v;
          lat[rb][i] = ok ? ls[i] : 0.f;
          mx = fmaxf(mx, v);
        }
      }
      mx = max_xor16_32(mx);               // this wave's 32 tokens, head r
      if (g == 0) xmax[w][r] = mx;
      __syncthreads();                     // X2
      const float mt = fmaxf(fmaxf(xmax[0][r], xmax[1][r]), fmaxf(xmax[2][r], xmax[3][r]));
      const bool need = mt > m_run + kTau;
      if (__ballot(need)) {
        const float m_new = need ? mt : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] *= alpha;
        l_sum *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      // P, its sum, and P' = P * token scale as two e4m3 terms under this block's exponent
      float pm = 0.f;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(p[rb][i] - m_use);
          l_sum += e;
          p[rb][i] = e * lat[rb][i];
          pm = fmaxf(pm, p[rb][i]);
        }
      pm = max_xor16_32(pm);
      const int ep = f8_exp(pm);
      const float sp = __uint_as_float((uint32_t)(127 - ep) << 23);
      if (g == 0) xexp[w][r] = ep;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float x4[4] = {p[rb][0] * sp, p[rb][1] * sp, p[rb][2] * sp, p[rb][3] * sp};
        uint32_t hi, lo;
        f8_split4(x4, hi, lo);
        const int c = 2 * w + rb;          // token chunk of 32 w + 16 rb, byte 4 g
        *reinterpret_cast<uint32_t*>(pex + pex_off(0, r, c) + 4 * g) = hi;
        *reinterpret_cast<uint32_t*>(pex + pex_off(1, r, c) + 4 * g) = lo;
      }
      __syncthreads();                     // X3
      // ---- values: B = P'' (lane: head r, tokens 16 g + 0..15 and 64 + 16 g + 0..15)
      const u32x4 b0 = *reinterpret_cast<const u32x4*>(pex + pex_off(0, r, g));
      const u32x4 b1 = *reinterpret_cast<const u32x4*>(pex + pex_off(0, r, 4 + g));
      const u32x4 c0 = *reinterpret_cast<const u32x4*>(pex + pex_off(1, r, g));
      const u32x4 c1 = *reinterpret_cast<const u32x4*>(pex + pex_off(1, r, 4 + g));
      const int32x8 ph = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
      const int32x8 pl = {(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
      const int eb = xexp[g][r];           // block g = compute wave g's tokens
      const int sp_hi = 127 + eb, sp_lo = 127 + eb - 4;
      // A = V^T: lane 16 g + 2 j + h addresses row (token) base_q + j, byte 8 h of
      // the feature chunk; the four reads take tokens 16 g + 0..7, + 8..15,
      // 64 + 16 g + 0..7, + 8..15.  Row offsets are formed here from an opaque
      // copy of the lane index, so that the compiler keeps four bases live, not
      // thirty-two addresses.
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int jj = (ln & 15) >> 1, hh = ln & 1, gq = ln >> 4;
      uint32_t vbase[4], vswz[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = 64 * (q >> 1) + 16 * gq + 8 * (q & 1) + jj;
        vbase[q] = row * kRowF8 + 128 * w + 8 * hh;
        vswz[q] = 16 * f8_swz(row);
      }
      auto vread = [&](int fb) {
        int32x2 v4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v4[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) int32x2*)((lds_char*)buf + vbase[q] + ((16u * fb) ^ vswz[q])));
        return int32x8{v4[0][0], v4[0][1], v4[1][0], v4[1][1], v4[2][0], v4[2][1], v4[3][0], v4[3][1]};
      };
      int32x8 va = vread(0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int fb = 0; fb < 8; ++fb) {
        int32x8 vn = va;
        if (fb + 1 < 8) vn = vread(fb + 1);     // the next block's operand, read under this block's products
        o[fb] = mfma_f8(va, ph, o[fb], 127, sp_hi);
        o[fb] = mfma_f8(va, pl, o[fb], 127, sp_lo);
        va = vn;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (n_tiles & 1) {                     // the staging waves' idle step
      __syncthreads();
      __syncthreads();
      __syncthreads();
    }
  }

  // ---- the heads' sums over the four waves' tokens, then o_part and lse
  l_sum += __shfl_xor(l_sum, 16, 64);
  l_sum += __shfl_xor(l_sum, 32, 64);
  if (g == 0) xmax[w][r] = l_sum;
  __syncthreads();
  const float l = xmax[0][r] + xmax[1][r] + xmax[2][r] + xmax[3][r];
  const float inv = l > 0.f ? 1.f / l : 0.f;
  uint16_t* op = a.o_part + ((int64_t)it.out_row * 16 + r) * kDc + 128 * w + 4 * g;
#pragma unroll
  for (int fb = 0; fb < 8; ++fb)
    *reinterpret_cast<half4*>(op + 16 * fb) = __builtin_convertvector(o[fb] * inv, half4);   // nearest even
  if (w == 0 && g == 0) a.lse_part[(int64_t)it.out_row * 16 + r] = l > 0.f ? (m_run + __log2f(l)) * kLn2 : -INFINITY;
}

// ===========================================================================
// H = 128, bf16 cache: eight waves per work-group, two per SIMD
// ===========================================================================
// A single wave per SIMD (decode_h128 above) leaves the matrix cores idle
// while it runs its softmax, its staging and its barriers.  Here each SIMD
// holds one score wave (waves 0-3) and one value wave (waves 4-7), and every
// 32-token tile takes two phases separated by barriers:
//   phase 1  score wave w: S^T for heads 32w..32w+31 over all 576 columns (36 x
//            mfma 32x32x16; K from the LDS tile; Q^T of the first kQReg2
//            k-steps in VGPRs, the rest from LDS), softmax against the fixed
//            reference maximum, P^T (fp16) to the exchange buffer;
//            value wave w: widens and stores its share of the next tile (four of
//            the nine 16-byte chunks per row), then issues the loads of the tile
//            after it;
//   phase 2  O^T += V^T . P^T: score wave w for features 128w..128w+31 (8
//            MFMAs, with its share of the staging (five chunks per row) woven
//            between them), value wave w for features 128w+32..128w+127 (24
//            MFMAs).
// The registers of one SIMD hold O^T for 128 features of all heads (256 per
// lane), 20 k-steps of Q^T for 32 heads (80) and one tile in flight (36): one
// wave alone could not hold more, two waves can split it so that each stays
// within 256.  With eight waves the LDS also serves about twice the bytes per
// clock that four waves draw from it.
// Q^T k-steps from kQReg2 on live in LDS as the register image of the score
// waves: the B-operand fragment of score wave w for tail k-step j is 64 lanes x
// 16 B, lane l at 16 l (so every fragment read is one contiguous, conflict-free
// 1 KB).
constexpr int kQReg2 = 18, kQTail2 = kDk / 16 - kQReg2;
constexpr int kQTail2Bytes = 4 * kQTail2 * 1024;          // 73,728 B
__device__ __forceinline__ uint32_t qtail2_off(int w, int j, int lane) { return ((w * kQTail2 + j) * 64 + lane) * 16; }

// Staging of a bf16 tile: work-group threads (tid & 255) own token (tid & 255) >> 3
// of the 32 and 16-byte chunks c8 + 8k of its row, c8 = tid & 7; this part holds
// chunks K0 <= k < K1.
template <int K0, int K1>
struct StageBf16 {
  static constexpr int kN = K1 - K0;
  u32x4 r[kN];
  const uint8_t* src;
  __device__ __forceinline__ void begin(const DecodeArgs& a, int64_t page, int t0, int t_end) {
    const int lt = threadIdx.x & 255, tok = lt >> 3;
    const bool ok = page >= 0 && t0 + tok < t_end;
    src = page_base(a, page, ok, kBlock * kRowBytesBf16) + ((t0 % kBlock) + tok) * kRowBytesBf16 + 16 * (lt & 7);
  }
  template <int I>
  __device__ __forceinline__ void load() { r[I] = ld16_stream(src + 128 * (K0 + I)); }
  __device__ __forceinline__ void load_all() {
#pragma unroll
    for (int i = 0; i < kN; ++i) r[i] = ld16_stream(src + 128 * (K0 + i));
  }
  template <int I>
  __device__ __forceinline__ void store(char* buf) {
    const int lt = threadIdx.x & 255;
    *reinterpret_cast<u32x4*>(buf + swz<kSwz128>(lt >> 3, lt & 7) + 128 * (K0 + I)) = bf16x8_to_f16x8(r[I]);
  }
  __device__ __forceinline__ void store_all(char* buf) {
    const int lt = threadIdx.x & 255;
    char* dst = buf + swz<kSwz128>(lt >> 3, lt & 7);
#pragma unroll
    for (int i = 0; i < kN; ++i) *reinterpret_cast<u32x4*>(dst + 128 * (K0 + i)) = bf16x8_to_f16x8(r[i]);
  }
};
constexpr int kStageSplit = 6;              // score waves stage chunks 0..5, value waves 6..8
using StageA = StageBf16<0, kStageSplit>;
using StageB = StageBf16<kStageSplit, 9>;

// Score chain of one tile for a score wave, as fenced steps (see H128Scores).
template <int kPf>
struct ScoresV2 {
  const char* buf;
  const char* qtail;
  const H128Lane& L;
  const half8 (&q)[kQReg2];
  floatx16 sacc;
  half8 kb[kPf], qb[kPf];
  static constexpr int kSteps = kDk / 16;

  __device__ __forceinline__ half8 kread(int ks) const {
    return *reinterpret_cast<const half8*>(buf + L.qk_off[ks & 3] + 128 * (ks >> 2));
  }
  template <int KS>
  __device__ __forceinline__ void step() {
    if constexpr (KS < kQReg2) sacc = mfma32x32x16(kb[KS % kPf], q[KS], sacc);
    else sacc = mfma32x32x16(kb[KS % kPf], qb[KS % kPf], sacc);
    constexpr int kn = KS + kPf;
    if constexpr (kn < kSteps) {
      kb[KS % kPf] = kread(kn);
      if constexpr (kn >= kQReg2) qb[KS % kPf] = *reinterpret_cast<const half8*>(qtail + 1024 * (kn - kQReg2));
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (KS + 1 < kSteps) step<KS + 1>();
  }
  __device__ __forceinline__ floatx16 run() {
    __builtin_amdgcn_sched_barrier(0);
    sacc = floatx16{};
#pragma unroll
    for (int d = 0; d < kPf; ++d) kb[d] = kread(d);
    static_assert(kQReg2 >= kPf, "the first Q^T fragments come from VGPRs");
    __builtin_amdgcn_sched_barrier(0);
    step<0>();
    return sacc;
  }
};

// Scores and softmax of one tile for a score wave (modes as h128_scores).  The
// maximum is taken over the unscaled scores and scaled once (scale_log2 > 0, so
// it is the maximum of the scaled scores), and the scale goes into the
// exponent's argument as one fused multiply-add.
template <int kMode>
__device__ __forceinline__ void v2_scores(const char* buf, const char* qtail, const H128Lane& L,
                                          const half8 (&q)[kQReg2], float& m_ref, float& l_sum,
                                          bool& overflow, int t0, int t_end, bool page_ok, float scale_log2,
                                          half8 (&p)[2]) {
  floatx16 sacc = ScoresV2<3>{buf, qtail, L, q}.run();
  if (!page_ok || t0 + kTile128 > t_end) {          // partial tile: mask the missing rows
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tt = t0 + 8 * (r >> 2) + 4 * L.g + (r & 3);
      if (!page_ok || tt >= t_end) sacc[r] = -INFINITY;
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
  mx = max_xor32(mx) * scale_log2;         // lanes l and l^32 hold the same head
  if (kMode == 1) {
    m_ref = fmaxf(m_ref, mx);
    return;
  }
  if (kMode == 0) {
    if (m_ref == -INFINITY) m_ref = mx;    // first non-empty tile: nothing accumulated yet
    overflow |= mx > m_ref + kTauFixed;
  }
  const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], scale_log2, -m_use));
    psum += e;
    p[r >> 3][r & 7] = (_Float16)e;
  }
  l_sum += psum;
}

// Value product of one tile for kNF feature blocks F0.. of SIMD slot w (block
// 4w + f covers features 128w + 32f .. +31) and all 128 heads: MFMA
// I = 4 kNF j + kNF hg + f over token half j and head group hg.  V^T fragments
// of one token half are held at a time (refilled right after their last use),
// P^T fragments two at a time.  With kStage, the score wave's share of the
// next tile is stored (and its registers reloaded from the tile after it)
// between the MFMAs, one chunk per step.
template <int kNF, int F0, bool kStage>
struct ValuesV2 {
  const char* buf;
  const char* pbuf;
  const H128Lane& L;
  int w;
  floatx16 (&o)[4 * kNF];
  StageA* st;
  char* nxt;
  half8 vb[kNF];
  half8 pt[2];
  static constexpr int kMfma = 8 * kNF;

  __device__ __forceinline__ half8 vread(int j, int f) const {
    const int blk = 4 * w + F0 + f;
    const uint32_t off = 16 * j * kRowLds + 128 * (blk >> 1);
    const half4 lo = lds_read_tr(buf, L.pv_off[blk & 1] + off);
    const half4 hi = lds_read_tr(buf, L.pv_off[2 + (blk & 1)] + off);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  __device__ __forceinline__ half8 pread(int j, int hg) const {
    return *reinterpret_cast<const half8*>(pbuf + hg * 32 * kPRow + L.p_off(j));
  }
  template <int I>
  __device__ __forceinline__ void step() {
    constexpr int j = I / (4 * kNF), hg = (I / kNF) % 4, f = I % kNF;
    o[4 * f + hg] = mfma32x32x16(vb[f], pt[hg & 1], o[4 * f + hg]);
    if constexpr (j == 0 && hg == 3) vb[f] = vread(1, f);          // last use of this token half's V^T
    if constexpr (f == kNF - 1 && I + 1 + kNF < kMfma) {           // P^T two head groups on, same slot
      constexpr int n2 = I + 1 + kNF, j2 = n2 / (4 * kNF), hg2 = (n2 / kNF) % 4;
      pt[hg2 & 1] = pread(j2, hg2);
    }
    if constexpr (kStage && I < StageA::kN) {
      st->template store<I>(nxt);
      __builtin_amdgcn_sched_barrier(0);     // the reload may not overtake the store of the same registers
      st->template load<I>();
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (I + 1 < kMfma) step<I + 1>();
  }
  __device__ __forceinline__ void run() {
    static_assert(!kStage || StageA::kN <= kMfma, "staging must fit in the value product");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < kNF; ++f) vb[f] = vread(0, f);
    pt[0] = pread(0, 0);
    pt[1] = pread(0, 1);
    __builtin_amdgcn_sched_barrier(0);
    step<0>();
  }
};

// Both kinds of wave walk the same segments and tiles and pass the same
// barriers: per segment two (table refill), per tile two (X1: tile s complete,
// the other buffer and the P buffer free; X2: P of all heads written).
struct SegV2 {
  int seg0, seg1, n_tiles;
};
// filled: the table already holds this segment (the kernel's prologue fills
// the first one); the two barriers are passed either way.
__device__ __forceinline__ SegV2 v2_segment(const DecodeArgs& a, const ItemRange& it, int seg0, int32_t* ptab,
                                            bool filled = false) {
  SegV2 sg;
  sg.seg0 = seg0;
  sg.seg1 = seg0 + min(it.t_end - seg0, kSegPages * kBlock);
  __syncthreads();                         // earlier users of the buffers and the table are done
  if (!filled) fill_ptab(a, it.b, sg.seg0, sg.seg1, ptab);
  __syncthreads();
  sg.n_tiles = (sg.seg1 - sg.seg0 + kTile128 - 1) / kTile128;
  return sg;
}
__device__ __forceinline__ int64_t v2_page(const SegV2& sg, const int32_t* ptab, int t) {
  const int pg = ptab[(min(t, sg.n_tiles - 1) * kTile128) / kBlock];   // read clamped, then select
  return t < sg.n_tiles ? pg : -1;
}

// Score waves: scores, softmax and P in phase 1; feature block 4w of the value
// product with their share of the staging in phase 2.
template <int kMode>
__device__ __forceinline__ void v2_score_pass(const DecodeArgs& a, const ItemRange& it, char* lds0, char* lds1,
                                              char* pbuf, const char* qtail, int32_t* ptab, const H128Lane& L,
                                              int w, const half8 (&q)[kQReg2], floatx16 (&oa)[4], float& m_ref,
                                              float& l_sum, bool& overflow) {
  const char* qimg = qtail + qtail2_off(w, 0, 32 * L.g + L.hl);
  for (int seg0 = it.t_begin; seg0 < it.t_end; seg0 += kSegPages * kBlock) {
    const SegV2 sg = v2_segment(a, it, seg0, ptab, kMode == 0 && seg0 == it.t_begin);
    StageA sa;
    sa.begin(a, v2_page(sg, ptab, 0), sg.seg0, sg.seg1);
    sa.load_all();
    sa.store_all(lds0);
    sa.begin(a, v2_page(sg, ptab, 1), sg.seg0 + kTile128, sg.seg1);
    sa.load_all();
    auto tile = [&](int s, const char* cur, char* nxt) {
      __syncthreads();                     // X1
      int pg0 = __builtin_amdgcn_readfirstlane((int)v2_page(sg, ptab, s));
      int pg2 = __builtin_amdgcn_readfirstlane((int)v2_page(sg, ptab, s + 2));
      asm volatile("" : "+s"(pg0), "+s"(pg2));
      half8 p[2];
      v2_scores<kMode>(cur, qimg, L, q, m_ref, l_sum, overflow, sg.seg0 + s * kTile128, sg.seg1, pg0 >= 0,
                       a.scale_log2, p);
      if (kMode != 1) {
        char* pw = pbuf + w * 32 * kPRow;
        *reinterpret_cast<half8*>(pw + L.p_off(0)) = p[0];
        *reinterpret_cast<half8*>(pw + L.p_off(1)) = p[1];
      }
      __syncthreads();                     // X2
      sa.begin(a, pg2, sg.seg0 + (s + 2) * kTile128, sg.seg1);   // the reloads read the tile after next
      if (kMode != 1) {
        ValuesV2<1, 0, true>{cur, pbuf, L, w, oa, &sa, nxt}.run();
      } else {
        sa.store_all(nxt);
        sa.load_all();
      }
    };
    for (int s = 0; s < sg.n_tiles; s += 2) {
      tile(s, lds0, lds1);
      if (s + 1 < sg.n_tiles) tile(s + 1, lds1, lds0);
    }
  }
}

// Value waves: their share of the staging in phase 1; feature blocks 4w + 1..3
// of the value product in phase 2.
template <int kMode>
__device__ __forceinline__ void v2_value_pass(const DecodeArgs& a, const ItemRange& it, char* lds0, char* lds1,
                                              const char* pbuf, int32_t* ptab, const H128Lane& L, int w,
                                              floatx16 (&ob)[12]) {
  for (int seg0 = it.t_begin; seg0 < it.t_end; seg0 += kSegPages * kBlock) {
    const SegV2 sg = v2_segment(a, it, seg0, ptab, kMode == 0 && seg0 == it.t_begin);
    StageB sb;
    sb.begin(a, v2_page(sg, ptab, 0), sg.seg0, sg.seg1);
    sb.load_all();
    sb.store_all(lds0);
    sb.begin(a, v2_page(sg, ptab, 1), sg.seg0 + kTile128, sg.seg1);
    sb.load_all();
    auto tile = [&](int s, const char* cur, char* nxt) {
      __syncthreads();                     // X1
      int pg2 = __builtin_amdgcn_readfirstlane((int)v2_page(sg, ptab, s + 2));
      asm volatile("" : "+s"(pg2));
      sb.store_all(nxt);
      sb.begin(a, pg2, sg.seg0 + (s + 2) * kTile128, sg.seg1);
      sb.load_all();
      __syncthreads();                     // X2
      if (kMode != 1) ValuesV2<3, 1, false>{cur, pbuf, L, w, ob, nullptr, nullptr}.run();
    };
    for (int s = 0; s < sg.n_tiles; s += 2) {
      tile(s, lds0, lds1);
      if (s + 1 < sg.n_tiles) tile(s + 1, lds1, lds0);
    }
  }
}

// The epilogue stages the normalised O^T of all 128 heads in LDS as fp16 rows
// (head h: 1 KB at 1024 h, its 16-byte chunk c at 16 (c ^ (h & 15)) so that the
// accumulators' writes spread over the banks), then the work-group stores whole
// rows of o_part: store k of wave v writes row 8 k + v, one 16-byte chunk a lane.
constexpr int kORows = 128 * 1024;
template <int kN>
__device__ __forceinline__ void v2_stage_o(char* orow, const floatx16 (&o)[kN], int feat0, const float (&inv)[4],
                                           int hl, int g) {
#pragma unroll
  for (int i = 0; i < kN; ++i) {
    const int f = i / 4, hg = i % 4, h = 32 * hg + hl;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const floatx4 x = floatx4{o[i][4 * rr], o[i][4 * rr + 1], o[i][4 * rr + 2], o[i][4 * rr + 3]} * inv[hg];
      const int c = (feat0 + 32 * f + 8 * rr) >> 3;
      *reinterpret_cast<half4*>(orow + 1024 * h + 16 * (c ^ (h & 15)) + 8 * g) =
          __builtin_convertvector(x, half4);   // round to nearest even
    }
  }
}
__device__ __forceinline__ void v2_store_rows(const DecodeArgs& a, const ItemRange& it, const char* orow) {
  const int lane = threadIdx.x & 63, v = threadIdx.x >> 6;
  uint16_t* dst = a.o_part + (int64_t)it.out_row * 128 * kDc;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int h = 8 * k + v;
    const u32x4 x = *reinterpret_cast<const u32x4*>(orow + 1024 * h + 16 * (lane ^ (h & 15)));
    *reinterpret_cast<u32x4*>(dst + h * kDc + 8 * lane) = x;
  }
}

__global__ __launch_bounds__(512, 1) void decode_h128v2(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kBuf128 + kPBuf + kQTail2Bytes + 4 * kSegPages];
  char* const lds0 = smem;
  char* const lds1 = smem + kBuf128;
  char* const pbuf = smem + 2 * kBuf128;
  char* const qtail = pbuf + kPBuf;
  int32_t* const ptab = reinterpret_cast<int32_t*>(qtail + kQTail2Bytes);
  static_assert(kORows <= 2 * kBuf128 + kPBuf + kQTail2Bytes, "the O rows fit below the page table");
  ItemRange it = item_range(a);
  if (!it.ok) return;
  if (a.num_pages <= 0) it.t_end = it.t_begin;     // no page can be valid (the loaders need page 0)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool scorer = wave < 4;                    // uniform per wave
  const int w = wave & 3;
  const int lane = threadIdx.x & 63, hl = lane & 31, g = lane >> 5;
  const H128Lane L = h128_lane();

  // Prologue, as one memory round trip: the Q^T k-steps from kQReg2 on (all
  // heads, to LDS: thread -> head tid / 4 and the 16-byte chunks c = tid % 4 + 4 i
  // of its row's tail; chunk c is k-step kQReg2 + c / 2, lane group c % 2), the
  // score waves' Q^T registers (loaded just before this, in their branch), and
  // the page table of the item's first segment (the first segment of pass 0
  // then skips its fill) are all requested before any of them is used.
  auto prologue = [&]() {
    const int hr = threadIdx.x >> 2;
    const uint16_t* qr = a.q_abs + ((int64_t)it.b * 128 + hr) * kDk + 16 * kQReg2;
    u32x4 qt[2 * kQTail2 / 4];
#pragma unroll
    for (int i = 0; i < 2 * kQTail2 / 4; ++i) qt[i] = ld16(qr + 8 * ((threadIdx.x & 3) + 4 * i));
    const int seg1 = it.t_begin + min(it.t_end - it.t_begin, kSegPages * kBlock);
    const int n0 = (seg1 - it.t_begin + kBlock - 1) / kBlock;          // <= kSegPages = 2 x 512
    const int i0 = threadIdx.x, i1 = threadIdx.x + 512;
    const int32_t p0 = i0 < n0 ? (int32_t)page_of(a, it.b, it.t_begin + i0 * kBlock) : -1;
    const int32_t p1 = i1 < n0 ? (int32_t)page_of(a, it.b, it.t_begin + i1 * kBlock) : -1;
#pragma unroll
    for (int i = 0; i < 2 * kQTail2 / 4; ++i) {
      const int c = (threadIdx.x & 3) + 4 * i;
      *reinterpret_cast<u32x4*>(qtail + qtail2_off(hr >> 5, c >> 1, (hr & 31) + 32 * (c & 1))) = qt[i];
    }
    if (i0 < n0) ptab[i0] = p0;
    if (i1 < n0) ptab[i1] = p1;
  };
  static_assert(kSegPages <= 2 * 512, "the prologue fills the first segment's table with two entries per thread");
  float m_ref = -INFINITY, l_sum = 0.f;
  bool overflow = false;
  float* red = reinterpret_cast<float*>(ptab);      // the table is not read after the passes
  if (scorer) {
    // Q^T as the B operand: lane holds q_abs[b][32w + hl][16 ks + 8 g .. +7] for the first kQReg2 k-steps.
    half8 q[kQReg2];
    const uint16_t* qp = a.q_abs + ((int64_t)it.b * 128 + 32 * w + hl) * kDk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kQReg2; ++ks) q[ks] = __builtin_bit_cast(half8, ld16(qp + 16 * ks));
    prologue();
    wait_vm<0>();                          // the Q loads retire before the tile loop's loads are issued
    floatx16 oa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) oa[i] = floatx16{};
    v2_score_pass<0>(a, it, lds0, lds1, pbuf, qtail, ptab, L, w, q, oa, m_ref, l_sum, overflow);
    if (__syncthreads_or(overflow)) {
      // Rare: some head's scores grew by more than 2^15 after its first tile.
      m_ref = -INFINITY;
      v2_score_pass<1>(a, it, lds0, lds1, pbuf, qtail, ptab, L, w, q, oa, m_ref, l_sum, overflow);
#pragma unroll
      for (int i = 0; i < 4; ++i) oa[i] = floatx16{};
      l_sum = 0.f;
      v2_score_pass<2>(a, it, lds0, lds1, pbuf, qtail, ptab, L, w, q, oa, m_ref, l_sum, overflow);
    }
    const float l_tot = l_sum + __shfl_xor(l_sum, 32, 64);
    __syncthreads();                       // every wave is done with the P buffer
    if (g == 0) red[32 * w + hl] = l_tot;
    __syncthreads();
    float inv[4];
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
      const float l = red[32 * hg + hl];
      inv[hg] = l > 0.f ? 1.f / l : 0.f;
    }
    v2_stage_o(smem, oa, 128 * w, inv, hl, g);
    if (g == 0)
      a.lse_part[(int64_t)it.out_row * 128 + 32 * w + hl] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    prologue();
    wait_vm<0>();
    floatx16 ob[12];
#pragma unroll
    for (int i = 0; i < 12; ++i) ob[i] = floatx16{};
    v2_value_pass<0>(a, it, lds0, lds1, pbuf, ptab, L, w, ob);
    if (__syncthreads_or(false)) {
      v2_value_pass<1>(a, it, lds0, lds1, pbuf, ptab, L, w, ob);
#pragma unroll
      for (int i = 0; i < 12; ++i) ob[i] = floatx16{};
      v2_value_pass<2>(a, it, lds0, lds1, pbuf, ptab, L, w, ob);
    }
    __syncthreads();
    __syncthreads();
    float inv[4];
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
      const float l = red[32 * hg + hl];
      inv[hg] = l > 0.f ? 1.f / l : 0.f;
    }
    v2_stage_o(smem, ob, 128 * w + 32, inv, hl, g);
  }
  __syncthreads();                         // every O row staged
  v2_store_rows(a, it, smem);
}

// ---------------------------------------------------------------------------
using H16Bf16 = LoaderBf16Wide<kSwz16, 256>;   // the staging waves are threads 256..511
using H16Int8 = LoaderInt8Wide<kSwz16, 256>;
using H16Int4 = LoaderInt4Wide<kSwz16, 256>;
using H16Int4Sym = LoaderInt4Wide<kSwz16, 256, true>;
using H16Int8Tok = LoaderInt8Wide<kSwz16, 256, true>;
using H16Int4SymK4 = LoaderInt4Wide<kSwz16, 256, true, true>;
using H16Int8c = LoaderInt8cWide<kSwz16, 256>;
using H16Int8cOpen = LoaderInt8cOpenWide<kSwz16, 256>;

hipError_t launch_decode_attn(const DecodeArgs& a, int num_heads, int cache_dtype, hipStream_t stream) {
  if (a.n_items <= 0) return hipSuccess;
  const dim3 grid(a.n_items), block(256);
  if (num_heads == 128) {
    if (cache_dtype == 0) hipLaunchKernelGGL(decode_h128v2, grid, dim3(512), 0, stream, a);
    else if (cache_dtype == 1) hipLaunchKernelGGL(decode_h128<1>, grid, block, 0, stream, a);
    else if (cache_dtype == 2) hipLaunchKernelGGL(decode_h128<2>, grid, block, 0, stream, a);
    else if (cache_dtype == 3) hipLaunchKernelGGL(decode_h128<3>, grid, block, 0, stream, a);
    else if (cache_dtype == 4) hipLaunchKernelGGL(decode_h128<4>, grid, block, 0, stream, a);
    else if (cache_dtype == 5) hipLaunchKernelGGL(decode_h128<5>, grid, block, 0, stream, a);
    else if (cache_dtype == 6) hipLaunchKernelGGL(decode_h128<6>, grid, block, 0, stream, a);
    else if (cache_dtype == 7) hipLaunchKernelGGL(decode_h128<7>, grid, block, 0, stream, a);
    else return hipErrorInvalidValue;
  } else if (num_heads == 16) {
    const dim3 block16(512);                       // 4 compute + 4 staging waves
    if (cache_dtype == 0) hipLaunchKernelGGL(decode_h16<H16Bf16>, grid, block16, 0, stream, a);
    else if (cache_dtype == 1) hipLaunchKernelGGL(decode_h16<H16Int8>, grid, block16, 0, stream, a);
    else if (cache_dtype == 2) hipLaunchKernelGGL(decode_h16<H16Int4>, grid, block16, 0, stream, a);
    else if (cache_dtype == 3) hipLaunchKernelGGL(decode_h16<H16Int4Sym>, grid, block16, 0, stream, a);
    else if (cache_dtype == 4) hipLaunchKernelGGL(decode_h16<H16Int8Tok>, grid, block16, 0, stream, a);
    else if (cache_dtype == 5) hipLaunchKernelGGL(decode_h16f8, grid, block16, 0, stream, a);
    else if (cache_dtype == 6) hipLaunchKernelGGL(decode_h16<H16Int4SymK4>, grid, block16, 0, stream, a);
    else if (cache_dtype == 7) hipLaunchKernelGGL((decode_h16<H16Int8c, H16Int8cOpen>), grid, block16, 0, stream, a);
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
