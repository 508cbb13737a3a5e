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
//     LDS in tiles of fp16 rows (1,152 B, 16-byte chunks XOR-swizzled by row).
//   * H = 128: wave w owns heads 32w..32w+31 and the whole 32-token tile:
//       S^T[32 tok x 32 head] = K[32 x 576] . Q^T    36 x mfma 32x32x16 (K from LDS,
//                                                     Q resident in VGPRs)
//       O^T[512 x 32 head] += V^T . P^T               32 x mfma 32x32x16 (V^T read from
//                                                     the same row-major tile with
//                                                     ds_read_b64_tr_b16; P^T is the
//                                                     score accumulator's own layout)
//     so all 128 heads share each LDS read of the latent.  bf16 tiles arrive by
//     direct global->LDS loads (no VGPRs) into a 4-tile ring and are widened to
//     fp16 in place by the lane that loaded them; two tiles stay in flight.
//   * H = 16: each wave takes 16 tokens of a 64-token page for all 16 heads
//     (mfma 16x16x32 scores, 16x16x16 values); the four waves' (max, sum, O) are
//     merged through LDS at the end.
//   * Quantised tiles, and H = 16, use register prefetch one tile ahead and a
//     2-tile LDS ring.
//   * Softmax in the log2 domain.  H = 128 fixes each head's reference max at its
//     first non-empty tile and never rescales O inside the loop (P <= 2^15 fits
//     fp16); if a later tile exceeds that by more than 2^15 the item is redone
//     against exact maxima (one scores-only pass, one accumulate pass).  H = 16
//     rescales lazily (only when the max grows by more than 2^8).
//   * Tokens past the item's end, or on pages whose id is outside the pool, are
//     zero-filled in LDS and masked to -inf.
#include <type_traits>

#include "common.h"
#include "decode_attn.h"

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
  const int L = max(a.seq_lens[it.seq], 0);
  const int pmax = min(it.first_page + it.n_pages, a.max_pages);
  r.t_begin = it.first_page * kBlock;
  r.t_end = min(pmax * kBlock, L);
  if (r.t_end < r.t_begin) r.t_end = r.t_begin;
  return r;
}

// Physical page of logical token t of sequence b, or -1 when out of range.
__device__ __forceinline__ int64_t page_of(const DecodeArgs& a, int b, int t) {
  const int lp = t / kBlock;
  if (lp >= a.max_pages) return -1;
  const int64_t p = a.block_table[(int64_t)b * a.max_pages + lp];
  return (p >= 0 && p < a.num_pages) ? p : -1;
}

// ===========================================================================
// Register-prefetch tile loaders: issue() loads a tile into registers, commit()
// writes it as fp16 rows into an LDS buffer.  kTok tokens (32 or 64), starting
// at a multiple of kTok within a page.  Thread tid owns token (tid >> 3) of each
// 32-token pass and the 16-byte output chunks (tid & 7) + 8k, k = 0..8 (k = 8 is
// the RoPE key), so all offsets are affine in k.  Rows past t_end and pages out
// of range become zeros.
// ===========================================================================
template <int kTok, int kSwz>
struct LoaderBf16Reg {
  static constexpr int kPass = kTok / 32;
  u32x4 r[9 * kPass];

  __device__ __forceinline__ void issue(const DecodeArgs& a, int b, int t0, int t_end) {
    const int64_t page = page_of(a, b, t0);
    const int tok = threadIdx.x >> 3;
    const uint8_t* base = a.pool + (page < 0 ? 0 : page) * (int64_t)(kBlock * kRowBytesBf16) +
                          (int64_t)((t0 % kBlock) + tok) * kRowBytesBf16 + 16 * (threadIdx.x & 7);
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const bool ok = page >= 0 && t0 + 32 * p + tok < t_end;
#pragma unroll
      for (int k = 0; k < 9; ++k)
        r[9 * p + k] = ok ? ld16_stream(base + 32 * p * kRowBytesBf16 + 128 * k) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void commit(char* lds_buf) const {
    const int tok = threadIdx.x >> 3;
    char* dst = lds_buf + swz<kSwz>(tok, threadIdx.x & 7);
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

// INT8 page: [64][576] codes | [64][16] f32 latent scales | [64][8] f32 key scales.
template <int kTok, int kSwz>
struct LoaderInt8Reg {
  static constexpr int kPass = kTok / 32;
  static constexpr int kPage = kBlock * 672;
  u32x2 c[9 * kPass];
  float s[9 * kPass];

  __device__ __forceinline__ void issue(const DecodeArgs& a, int b, int t0, int t_end) {
    const int64_t page = page_of(a, b, t0);
    const int tok = threadIdx.x >> 3, c8 = threadIdx.x & 7;
    const uint8_t* pg = a.pool + (page < 0 ? 0 : page) * (int64_t)kPage;
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int row = (t0 % kBlock) + 32 * p + tok;
      const bool ok = page >= 0 && t0 + 32 * p + tok < t_end;
      const uint8_t* codes = pg + row * 576 + 8 * c8;
      const float* cs = reinterpret_cast<const float*>(pg + 64 * 576) + row * 16 + (c8 >> 2);
      const float* ks = reinterpret_cast<const float*>(pg + 64 * 576 + 64 * 64) + row * 8 + c8;
#pragma unroll
      for (int k = 0; k < 9; ++k) {
        c[9 * p + k] = ok ? *reinterpret_cast<const u32x2*>(codes + 64 * k) : u32x2{0u, 0u};
        s[9 * p + k] = ok ? (k < 8 ? cs[2 * k] : ks[0]) : 0.f;
      }
    }
  }
  __device__ __forceinline__ void commit(char* lds_buf) const {
    const int tok = threadIdx.x >> 3;
    char* dst = lds_buf + swz<kSwz>(tok, threadIdx.x & 7);
#pragma unroll
    for (int p = 0; p < kPass; ++p)
#pragma unroll
      for (int k = 0; k < 9; ++k) {
        const _Float16 sh = (_Float16)s[9 * p + k];
        const half2v s2 = {sh, sh};
        const u32x2 lo = int8x4_to_f16(c[9 * p + k][0], s2), hi = int8x4_to_f16(c[9 * p + k][1], s2);
        *reinterpret_cast<u32x4*>(dst + 32 * p * kRowLds + 128 * k) = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
  }
};

// INT4 page: [64][256] latent nibbles | [64][64] int8 key codes | [64][16] f32 scales
//            | [64][16] f32 zeros | [64][8] f32 key scales.
template <int kTok, int kSwz>
struct LoaderInt4Reg {
  static constexpr int kPass = kTok / 32;
  static constexpr int kPage = kBlock * 480;
  uint32_t n[8 * kPass];     // 8 nibbles (latent chunk k) per dword
  u32x2 kc[kPass];           // 8 key codes (chunk 8)
  float s[9 * kPass];        // scale per chunk (k = 8: key scale)
  float z[8 * kPass];        // zero point per latent chunk

  __device__ __forceinline__ void issue(const DecodeArgs& a, int b, int t0, int t_end) {
    const int64_t page = page_of(a, b, t0);
    const int tok = threadIdx.x >> 3, c8 = threadIdx.x & 7;
    const uint8_t* pg = a.pool + (page < 0 ? 0 : page) * (int64_t)kPage;
    const float* scales = reinterpret_cast<const float*>(pg + 64 * 256 + 64 * 64);
    const float* zeros = scales + 64 * 16;
    const float* kscales = zeros + 64 * 16;
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
      const int row = (t0 % kBlock) + 32 * p + tok;
      const bool ok = page >= 0 && t0 + 32 * p + tok < t_end;
      const uint8_t* nib = pg + row * 256 + 4 * c8;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        n[8 * p + k] = ok ? *reinterpret_cast<const uint32_t*>(nib + 32 * k) : 0u;
        s[9 * p + k] = ok ? scales[row * 16 + 2 * k + (c8 >> 2)] : 0.f;
        z[8 * p + k] = ok ? zeros[row * 16 + 2 * k + (c8 >> 2)] : 0.f;
      }
      kc[p] = ok ? *reinterpret_cast<const u32x2*>(pg + 64 * 256 + row * 64 + 8 * c8) : u32x2{0u, 0u};
      s[9 * p + 8] = ok ? kscales[row * 8 + c8] : 0.f;
    }
  }
  __device__ __forceinline__ void commit(char* lds_buf) const {
    const int tok = threadIdx.x >> 3;
    char* dst = lds_buf + swz<kSwz>(tok, threadIdx.x & 7);
    const half2v bias = {(_Float16)-1024.0f, (_Float16)-1024.0f};
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const _Float16 sh = (_Float16)s[9 * p + k], zh = (_Float16)z[8 * p + k];
        const half2v s2 = {sh, sh}, z2 = {zh, zh};
        const uint32_t w = n[8 * p + k];
        u32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t byte = (w >> (8 * j)) & 0xffu;
          // (element 2j, element 2j+1) = (low nibble, high nibble) as fp16 1024 + q
          const uint32_t h = 0x64006400u | (byte & 0xfu) | ((byte >> 4) << 16);
          const half2v qv = __builtin_bit_cast(half2v, h) + bias;
          v[j] = __builtin_bit_cast(uint32_t, qv * s2 + z2);
        }
        *reinterpret_cast<u32x4*>(dst + 32 * p * kRowLds + 128 * k) = v;
      }
      const _Float16 kh = (_Float16)s[9 * p + 8];
      const half2v k2 = {kh, kh};
      const u32x2 lo = int8x4_to_f16(kc[p][0], k2), hi = int8x4_to_f16(kc[p][1], k2);
      *reinterpret_cast<u32x4*>(dst + 32 * p * kRowLds + 128 * 8) = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  }
};

// ===========================================================================
// H = 128
// ===========================================================================
constexpr int kTile128 = 32;
constexpr int kBuf128 = kTile128 * kRowLds;        // 36,864 B

struct H128Lane {
  uint32_t qk_off[4];     // score operand: row hl, chunk 2 ks + g
  uint32_t pv_off[4];     // transposed value read: row 4 g + (gi >> 2) + 8 hi (+16 j); [2 hi + parity]
  int g;
};

__device__ __forceinline__ H128Lane h128_lane() {
  H128Lane L;
  const int lane = threadIdx.x & 63;
  const int hl = lane & 31, g = lane >> 5, grp = lane >> 4, gi = lane & 15;
  L.g = g;
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

// One 32-token tile of work for one wave.  kMode 0: accumulate with a per-head
// reference max fixed at the head's first non-empty tile (sets `overflow` when a
// later tile exceeds it by more than kTauFixed); kMode 1: scores only, m_ref
// becomes the exact max; kMode 2: accumulate against the exact max in m_ref.
template <int kMode>
__device__ __forceinline__ void h128_tile(const char* buf, const H128Lane& L, const half8 (&q)[kDk / 16],
                                          floatx16 (&o)[16], float& m_ref, float& l_sum, bool& overflow,
                                          int t0, int t_end, bool page_ok, float scale_log2) {
  auto kread = [&](int ks) -> half8 {
    return *reinterpret_cast<const half8*>(buf + L.qk_off[ks & 3] + 128 * (ks >> 2));
  };
  floatx16 sacc = floatx16{};
  half8 k0 = kread(0), k1 = kread(1), k2 = kread(2);
#pragma unroll
  for (int ks = 0; ks < kDk / 16; ++ks) {
    const half8 kn = (ks + 3 < kDk / 16) ? kread(ks + 3) : k2;
    sacc = mfma32x32x16(k0, q[ks], sacc);
    k0 = k1;
    k1 = k2;
    k2 = kn;
  }
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
  mx = wave_max_xor(mx, 32);               // lanes l and l^32 hold the same head
  if (kMode == 1) {
    m_ref = fmaxf(m_ref, mx);
    return;
  }
  if (kMode == 0) {
    if (m_ref == -INFINITY) m_ref = mx;    // first non-empty tile: nothing accumulated yet
    overflow |= mx > m_ref + kTauFixed;
  }
  const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
  half8 p[2];
  float psum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float e = __builtin_amdgcn_exp2f(sacc[r] - m_use);
    psum += e;
    p[r >> 3][r & 7] = (_Float16)e;
  }
  l_sum += psum;
  // O^T += V^T . P^T: step i covers tokens 16 (i / 16) .. +15 and features
  // 32 (i % 16) .. +31; the transposed reads run two steps ahead of the MFMAs.
  auto vread = [&](int i) -> half8 {
    const int j = i >> 4, tile = i & 15;
    const uint32_t off = 16 * j * kRowLds + 128 * (tile >> 1);
    const half4 lo = lds_read_tr(buf, L.pv_off[tile & 1] + off);
    const half4 hi = lds_read_tr(buf, L.pv_off[2 + (tile & 1)] + off);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  half8 v0 = vread(0), v1 = vread(1);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const half8 vn = (i + 2 < 32) ? vread(i + 2) : v1;
    o[i & 15] = mfma32x32x16(v0, p[i >> 4], o[i & 15]);
    v0 = v1;
    v1 = vn;
  }
}

// ---- pipeline A: register prefetch, 2-tile ring (quantised formats) ----------
template <class Loader, int kMode>
__device__ __forceinline__ void h128_pass_reg(const DecodeArgs& a, const ItemRange& it, char* lds,
                                              const H128Lane& L, const half8 (&q)[kDk / 16], floatx16 (&o)[16],
                                              float& m_ref, float& l_sum, bool& overflow) {
  const int n_tiles = (it.t_end - it.t_begin + kTile128 - 1) / kTile128;
  Loader ld;
  if (n_tiles > 0) {
    ld.issue(a, it.b, it.t_begin, it.t_end);
    __syncthreads();                       // earlier users of the buffers are done
    ld.commit(lds);
    if (n_tiles > 1) ld.issue(a, it.b, it.t_begin + kTile128, it.t_end);
  }
  for (int s = 0; s < n_tiles; ++s) {
    __syncthreads();                       // tile s visible; buffer (s+1)&1 free
    if (s + 1 < n_tiles) {
      ld.commit(lds + ((s + 1) & 1) * kBuf128);
      if (s + 2 < n_tiles) ld.issue(a, it.b, it.t_begin + (s + 2) * kTile128, it.t_end);
    }
    const int t0 = it.t_begin + s * kTile128;
    h128_tile<kMode>(lds + (s & 1) * kBuf128, L, q, o, m_ref, l_sum, overflow, t0, it.t_end,
                     page_of(a, it.b, t0) >= 0, a.scale_log2);
  }
}

// ---- pipeline B: direct global->LDS loads, 4-tile ring (bf16) ----------------
// Wave w fills LDS bytes [9216 w, 9216 w + 9216) of a tile with 9 loads of
// 64 lanes x 16 B; the lane writing LDS offset o carries the global chunk
// (row = o / 1152, logical chunk = physical chunk ^ (row & 7)).  After its own
// loads have landed, each lane widens exactly those 16 bytes to fp16 in place
// (or zeroes them for rows past the end / bad pages), so no other lane's data
// is touched before the next barrier.
struct DmaBf16Tile {
  uint32_t loff;          // LDS byte offset of this lane's chunk 0 within a tile
  int wave;

  __device__ __forceinline__ void init() {
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    loff = 9216 * wave + 16 * (threadIdx.x & 63);
  }
  // Byte offset, from the tile's first cache row, of the chunk lane-slot k carries.
  __device__ __forceinline__ uint32_t goff(int k) const {
    const uint32_t o = loff + 1024 * k;
    const uint32_t row = o / kRowLds;
    const uint32_t pc = (o - row * kRowLds) >> 4;
    return row * kRowBytesBf16 + 16 * (pc ^ swz_key<kSwz128>((int)row));
  }
  // The load is issued through inline assembly so that the compiler does not
  // track it: otherwise it waits for every outstanding direct load before any
  // LDS read it cannot prove disjoint, which would serialise the ring.  The
  // waits are placed explicitly (wait_vm_tiles) instead.
  __device__ __forceinline__ void issue(const uint8_t* src, char* lds_tile) const {
    const uint32_t lds_base =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(lds_tile + 9216 * wave);
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      const uint8_t* g = src + goff(k);
      asm volatile(
          "s_mov_b32 m0, %1\n\t"
          "s_nop 0\n\t"
          "global_load_lds_dwordx4 %0, off"
          :
          : "v"(g), "s"(lds_base + 1024 * k)
          : "memory", "m0");
    }
  }
  __device__ __forceinline__ void convert(char* lds_tile, int valid_rows) const {
    u32x4 v[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) v[k] = *reinterpret_cast<const u32x4*>(lds_tile + loff + 1024 * k);
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      const uint32_t o = loff + 1024 * k;
      const int row = (int)(o / kRowLds);
      *reinterpret_cast<u32x4*>(lds_tile + o) = row < valid_rows ? bf16x8_to_f16x8(v[k]) : u32x4{0u, 0u, 0u, 0u};
    }
  }
};

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] = 7 |
// lgkmcnt[11:8] = 15 | vmcnt[5:4] in bits [15:14]).
template <int kN>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((kN & 15) | (7 << 4) | (15 << 8) | ((kN >> 4) << 14));
}
// Wait until this wave's loads for a tile have landed while `tiles_after` later
// tiles (9 loads each) may still be in flight.
__device__ __forceinline__ void wait_vm_tiles(int tiles_after) {
  if (tiles_after >= 2) wait_vm<18>();
  else if (tiles_after == 1) wait_vm<9>();
  else wait_vm<0>();
}

// The pages of an item are looked up from an LDS copy of its block-table slice,
// refreshed every kSegPages pages while no direct load is in flight, so the only
// vector-memory operations inside the pipeline are the tile loads themselves
// (the vmcnt accounting above relies on that).
constexpr int kSegPages = 2048;

template <int kMode>
__device__ __forceinline__ void h128_pass_dma(const DecodeArgs& a, const ItemRange& it, char* lds, int32_t* ptab,
                                              const H128Lane& L, const DmaBf16Tile& D, const half8 (&q)[kDk / 16],
                                              floatx16 (&o)[16], float& m_ref, float& l_sum, bool& overflow) {
  for (int seg0 = it.t_begin; seg0 < it.t_end; seg0 += kSegPages * kBlock) {
    const int seg1 = min(it.t_end, seg0 + kSegPages * kBlock);
    const int n_pages = (seg1 - seg0 + kBlock - 1) / kBlock;
    __syncthreads();                       // earlier users of the ring and the table are done
    for (int i = threadIdx.x; i < n_pages; i += 256) ptab[i] = (int32_t)page_of(a, it.b, seg0 + i * kBlock);
    __syncthreads();
    const int n_tiles = (seg1 - seg0 + kTile128 - 1) / kTile128;
    auto page_at = [&](int t) -> int { return ptab[(t * kTile128) / kBlock]; };
    auto tile_src = [&](int t) -> const uint8_t* {
      const int page = page_at(t);
      return a.pool + (int64_t)(page < 0 ? 0 : page) * (kBlock * kRowBytesBf16) +
             (int64_t)(((seg0 + t * kTile128) % kBlock) * kRowBytesBf16);
    };
    auto valid_rows = [&](int t) -> int {
      return page_at(t) >= 0 ? min(kTile128, seg1 - (seg0 + t * kTile128)) : 0;
    };
    const bool any_pages = a.num_pages > 0;
    if (any_pages) {
      for (int t = 0; t < min(3, n_tiles); ++t) D.issue(tile_src(t), lds + t * kBuf128);
    }
    wait_vm_tiles(any_pages ? min(2, n_tiles - 1) : 0);
    D.convert(lds, valid_rows(0));
    for (int s = 0; s < n_tiles; ++s) {
      __syncthreads();                     // tile s converted by all; tile s-1 no longer read
      if (s + 3 < n_tiles && any_pages) D.issue(tile_src(s + 3), lds + ((s + 3) & 3) * kBuf128);
      const int t0 = seg0 + s * kTile128;
      h128_tile<kMode>(lds + (s & 3) * kBuf128, L, q, o, m_ref, l_sum, overflow, t0, seg1, page_at(s) >= 0,
                       a.scale_log2);
      // Widen this lane's share of the next tile while the value MFMAs drain.
      if (s + 1 < n_tiles) {
        wait_vm_tiles(any_pages ? min(2, n_tiles - 1 - (s + 1)) : 0);
        D.convert(lds + ((s + 1) & 3) * kBuf128, valid_rows(s + 1));
      }
    }
    wait_vm<0>();
  }
}

template <int kCache>
__global__ __launch_bounds__(256, 1) void decode_h128(DecodeArgs a) {
  constexpr int kRing = (kCache == 0) ? 4 : 2;
  __shared__ __attribute__((aligned(16))) char lds[kRing * kBuf128];
  __shared__ int32_t ptab[kCache == 0 ? kSegPages : 1];
  const ItemRange it = item_range(a);
  if (!it.ok) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hl = lane & 31;
  const int g = lane >> 5;
  const int h = wave * 32 + hl;
  const H128Lane L = h128_lane();

  // Q^T as the B operand: lane holds q_abs[b][h][16 ks + 8 g .. +7].
  half8 q[kDk / 16];
  {
    const uint16_t* qp = a.q_abs + ((int64_t)it.b * 128 + h) * kDk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kDk / 16; ++ks) q[ks] = __builtin_bit_cast(half8, ld16(qp + 16 * ks));
  }
  floatx16 o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = floatx16{};
  float m_ref = -INFINITY, l_sum = 0.f;
  bool overflow = false;

  if constexpr (kCache == 0) {
    // Retire the Q loads before the first direct load: the compiler cannot see
    // the direct loads, so its own vmcnt waits for Q inside the loop would
    // otherwise also stall on tile loads.
    wait_vm<0>();
    DmaBf16Tile D;
    D.init();
    h128_pass_dma<0>(a, it, lds, ptab, L, D, q, o, m_ref, l_sum, overflow);
    if (__syncthreads_or(overflow)) {
      // Rare: some head's scores grew by more than 2^15 after its first tile.
      m_ref = -INFINITY;
      h128_pass_dma<1>(a, it, lds, ptab, L, D, q, o, m_ref, l_sum, overflow);
#pragma unroll
      for (int i = 0; i < 16; ++i) o[i] = floatx16{};
      l_sum = 0.f;
      h128_pass_dma<2>(a, it, lds, ptab, L, D, q, o, m_ref, l_sum, overflow);
    }
  } else {
    using Loader = typename std::conditional<kCache == 1, LoaderInt8Reg<kTile128, kSwz128>,
                                              LoaderInt4Reg<kTile128, kSwz128>>::type;
    h128_pass_reg<Loader, 0>(a, it, lds, L, q, o, m_ref, l_sum, overflow);
    if (__syncthreads_or(overflow)) {
      m_ref = -INFINITY;
      h128_pass_reg<Loader, 1>(a, it, lds, L, q, o, m_ref, l_sum, overflow);
#pragma unroll
      for (int i = 0; i < 16; ++i) o[i] = floatx16{};
      l_sum = 0.f;
      h128_pass_reg<Loader, 2>(a, it, lds, L, q, o, m_ref, l_sum, overflow);
    }
  }

  // ---- normalise and write the partial ----
  const float l_tot = l_sum + __shfl_xor(l_sum, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
  float* op = a.o_part + ((int64_t)it.out_row * 128 + h) * kDc + 4 * g;
#pragma unroll
  for (int tile = 0; tile < 16; ++tile) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      floatx4 v = {o[tile][4 * rr], o[tile][4 * rr + 1], o[tile][4 * rr + 2], o[tile][4 * rr + 3]};
      *reinterpret_cast<floatx4*>(op + 32 * tile + 8 * rr) = v * inv;
    }
  }
  if (g == 0) a.lse_part[(int64_t)it.out_row * 128 + h] = lse;
}

// ===========================================================================
// H = 16
// ===========================================================================
constexpr int kTile16 = 64;
constexpr int kBuf16 = kTile16 * kRowLds;          // 73,728 B

template <class Loader>
__global__ __launch_bounds__(256, 1) void decode_h16(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kBuf16];
  const ItemRange it = item_range(a);
  if (!it.ok) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hl = lane & 15;          // head (MFMA column)
  const int grp = lane >> 4;         // 0..3
  const int n_tiles = (it.t_end - it.t_begin + kTile16 - 1) / kTile16;

  // Q^T as the B operand of 16x16x32: lane holds q_abs[b][hl][32 ks + 8 grp .. +7].
  half8 q[kDk / 32];
  {
    const uint16_t* qp = a.q_abs + ((int64_t)it.b * 16 + hl) * kDk + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < kDk / 32; ++ks) q[ks] = __builtin_bit_cast(half8, ld16(qp + 32 * ks));
  }
  floatx4 o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = floatx4{};
  float m_run = -INFINITY;
  float l_sum = 0.f;

  Loader ld;
  if (n_tiles > 0) {
    ld.issue(a, it.b, it.t_begin, it.t_end);
    ld.commit(lds);
    if (n_tiles > 1) ld.issue(a, it.b, it.t_begin + kTile16, it.t_end);
  }

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

  for (int s = 0; s < n_tiles; ++s) {
    __syncthreads();
    if (s + 1 < n_tiles) {
      ld.commit(lds + ((s + 1) & 1) * kBuf16);
      if (s + 2 < n_tiles) ld.issue(a, it.b, it.t_begin + (s + 2) * kTile16, it.t_end);
    }
    const char* buf = lds + (s & 1) * kBuf16;
    const int t0 = it.t_begin + s * kTile16;
    const bool page_ok = page_of(a, it.b, t0) >= 0;

    floatx4 sacc = floatx4{};
#pragma unroll
    for (int ks = 0; ks < kDk / 32; ++ks) {
      const half8 kv = *reinterpret_cast<const half8*>(buf + qk_off[ks & 1] + 128 * (ks >> 1));
      sacc = mfma16x16x32(kv, q[ks], sacc);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tt = t0 + tw + 4 * grp + r;
      float v = sacc[r] * a.scale_log2;
      if (!page_ok || tt >= it.t_end) v = -INFINITY;
      sacc[r] = v;
      mx = fmaxf(mx, v);
    }
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
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

  // ---- merge the four waves (each saw a quarter of every page) ----
  float l_w = l_sum;
  l_w += __shfl_xor(l_w, 16, 64);
  l_w += __shfl_xor(l_w, 32, 64);
  __syncthreads();                                   // all waves done with the tiles
  float* red = reinterpret_cast<float*>(lds);        // [4][16][512] O, then [4][16] m, [4][16] l
  float* red_m = red + 4 * 16 * kDc;
  float* red_l = red_m + 64;
#pragma unroll
  for (int tile = 0; tile < 32; ++tile) {
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * 16 + hl) * kDc + 16 * tile + 4 * grp + r] = o[tile][r];
  }
  if (grp == 0) {
    red_m[wave * 16 + hl] = m_run;
    red_l[wave * 16 + hl] = l_w;
  }
  __syncthreads();
  {
    const int head = threadIdx.x >> 4;               // 0..15
    const int f0 = (threadIdx.x & 15) * 32;          // 32 features each
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
    float* op = a.o_part + ((int64_t)it.out_row * 16 + head) * kDc + f0;
#pragma unroll
    for (int f = 0; f < 32; f += 4) {
      floatx4 v = floatx4{};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const floatx4 x = *reinterpret_cast<const floatx4*>(red + (w * 16 + head) * kDc + f0 + f);
        v += ew[w] * x;
      }
      *reinterpret_cast<floatx4*>(op + f) = v * inv;
    }
    if ((threadIdx.x & 15) == 0)
      a.lse_part[(int64_t)it.out_row * 16 + head] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
using H16Bf16 = LoaderBf16Reg<kTile16, kSwz16>;
using H16Int8 = LoaderInt8Reg<kTile16, kSwz16>;
using H16Int4 = LoaderInt4Reg<kTile16, kSwz16>;

hipError_t launch_decode_attn(const DecodeArgs& a, int num_heads, int cache_dtype, hipStream_t stream) {
  if (a.n_items <= 0) return hipSuccess;
  const dim3 grid(a.n_items), block(256);
  if (num_heads == 128) {
    if (cache_dtype == 0) hipLaunchKernelGGL(decode_h128<0>, grid, block, 0, stream, a);
    else if (cache_dtype == 1) hipLaunchKernelGGL(decode_h128<1>, grid, block, 0, stream, a);
    else if (cache_dtype == 2) hipLaunchKernelGGL(decode_h128<2>, grid, block, 0, stream, a);
    else return hipErrorInvalidValue;
  } else if (num_heads == 16) {
    if (cache_dtype == 0) hipLaunchKernelGGL(decode_h16<H16Bf16>, grid, block, 0, stream, a);
    else if (cache_dtype == 1) hipLaunchKernelGGL(decode_h16<H16Int8>, grid, block, 0, stream, a);
    else if (cache_dtype == 2) hipLaunchKernelGGL(decode_h16<H16Int4>, grid, block, 0, stream, a);
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mla
