// decode_attn.hip -- split-KV absorbed MLA decode attention for gfx950.
//
// What is computed ("DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界" §2.2-§2.4 and
// §6.1; "手搓 MLA:从 MHA 到 weight absorption" §四): every query head of a sequence
// attends to the same cached rows [c_t (512) ; k_pe_t (64)], i.e. MQA with one
// shared "KV head" of width 576 for scores and 512 for values.  Per work item
// (a run of a sequence's pages) and head:
//   s_t = scale * q_abs . row_t,  o = sum_t e^{s_t-m} c_t / l,  lse = m + ln l.
//
// gfx950 design
//   * One work-group (4 wave64s, 256 threads) per work item; the item's tokens
//     are streamed through LDS in tiles.  All 256 threads load a tile from HBM
//     with coalesced 16-byte loads into registers one tile ahead, widen bf16 to
//     fp16 (exact), and store it row-major in LDS (double buffered).
//   * H = 128: wave w owns heads 32w..32w+31 and the whole 32-token tile.
//       scores S^T[32 tok x 32 head] = K[32 x 576] . Q^T       (36 x mfma 32x32x16;
//         K from LDS, Q resident in VGPRs)
//       O^T[512 x 32 head] += V^T[512 x 32 tok] . P^T           (32 x mfma 32x32x16;
//         V^T read straight from the row-major tile with ds_read_b64_tr_b16,
//         P^T is the score accumulator's own lane layout, rounded to fp16)
//     so every head of the sequence shares each LDS read of the latent.
//   * H = 16: each wave takes 16 tokens of a 64-token page for all 16 heads
//     (mfma 16x16x32 for scores, 16x16x16 for values); the four waves' running
//     (max, sum, O) are merged through LDS at the end.
//   * Online softmax in the log2 domain with a lazy running max: O and l are
//     only rescaled when a tile's max exceeds the reference max by more than
//     kTau (so P <= 2^kTau stays far inside fp16), which is exact after the
//     final division by l.
//   * Tokens past the item's end, or on pages whose id is outside the pool,
//     are zero-filled in LDS and masked to -inf.
#include "common.h"
#include "decode_attn.h"

namespace mla {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;        // lazy-rescale threshold (log2 units), H = 16
constexpr float kTauFixed = 15.0f;  // fixed-reference headroom (log2 units), H = 128: P <= 2^15

// LDS tile layout: fp16 rows of 576 (1,152 B = 72 chunks of 16 B), no padding;
// the 16-byte chunk index of row r is XORed with (r & 7) so that the eight rows
// read together by an MFMA operand fetch land in different banks.
constexpr int kRowLds = kDk * 2;                    // 1,152 B
constexpr int kChunksPerRow = kRowBytesBf16 / 16;   // 72 x 16 B per token row

__device__ __forceinline__ uint32_t swz(int row, int chunk) {
  return (uint32_t)(row * kRowLds + 16 * (chunk ^ (row & 7)));
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

// ---------------------------------------------------------------------------
// Tile loader, bf16 pool: kTok tokens (a multiple of 32 dividing 64) starting
// at token t0 -> registers (one tile ahead) -> fp16 rows in LDS.  Thread tid
// owns token (tid >> 3) of every 32-token pass and the 16-byte columns
// (tid & 7) + 8k, k = 0..8, so both the global and the LDS offsets are affine
// in k; a wave's load covers 8 tokens x 128 contiguous bytes.
// ---------------------------------------------------------------------------
template <int kTok>
struct LoaderBf16 {
  static constexpr int kPass = kTok / 32;
  static constexpr int kPer = 9 * kPass;          // 16-byte chunks per thread
  u32x4 r[kPer];

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
    char* dst = lds_buf + swz(tok, threadIdx.x & 7);
#pragma unroll
    for (int p = 0; p < kPass; ++p)
#pragma unroll
      for (int k = 0; k < 9; ++k)
        *reinterpret_cast<u32x4*>(dst + 32 * p * kRowLds + 128 * k) = bf16x8_to_f16x8(r[9 * p + k]);
  }
};

// ===========================================================================
// H = 128
// ===========================================================================
constexpr int kTile128 = 32;
constexpr int kBuf128 = kTile128 * kRowLds;        // 36,864 B

// One pass over the item's tiles.  kMode 0: accumulate with a per-head
// reference max fixed at the head's first non-empty tile, flagging `overflow`
// if a later tile's max exceeds it by more than kTauFixed; kMode 1: scores only,
// returning the exact per-head max in m_ref; kMode 2: accumulate with the exact
// max already in m_ref (no overflow possible).
template <int kMode>
__device__ __forceinline__ void h128_pass(const DecodeArgs& a, const ItemRange& it, char* lds,
                                          const half8 (&q)[kDk / 16], floatx16 (&o)[16],
                                          float& m_ref, float& l_sum, bool& overflow,
                                          const uint32_t (&qk_off)[4], const uint32_t (&pv_off)[2]) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const int n_tiles = (it.t_end - it.t_begin + kTile128 - 1) / kTile128;
  LoaderBf16<kTile128> ld;
  if (n_tiles > 0) {
    ld.issue(a, it.b, it.t_begin, it.t_end);
    __syncthreads();                       // previous users of the buffers are done
    ld.commit(lds);
    if (n_tiles > 1) ld.issue(a, it.b, it.t_begin + kTile128, it.t_end);
  }
  for (int s = 0; s < n_tiles; ++s) {
    __syncthreads();                       // tile s visible; buffer (s+1)&1 free
    if (s + 1 < n_tiles) {
      ld.commit(lds + ((s + 1) & 1) * kBuf128);
      if (s + 2 < n_tiles) ld.issue(a, it.b, it.t_begin + (s + 2) * kTile128, it.t_end);
    }
    const char* buf = lds + (s & 1) * kBuf128;
    const int t0 = it.t_begin + s * kTile128;
    const bool page_ok = page_of(a, it.b, t0) >= 0;

    // ---- scores S^T (token x head) ----
    floatx16 sacc = floatx16{};
#pragma unroll
    for (int ks = 0; ks < kDk / 16; ++ks) {
      const half8 kv = *reinterpret_cast<const half8*>(buf + qk_off[ks & 3] + 128 * (ks >> 2));
      sacc = mfma32x32x16(kv, q[ks], sacc);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tt = t0 + 8 * (r >> 2) + 4 * g + (r & 3);
      float v = sacc[r] * a.scale_log2;
      if (!page_ok || tt >= it.t_end) v = -INFINITY;
      sacc[r] = v;
      mx = fmaxf(mx, v);
    }
    mx = wave_max_xor(mx, 32);             // lanes l and l^32 hold the same head
    if (kMode == 1) {
      m_ref = fmaxf(m_ref, mx);
      continue;
    }
    if (kMode == 0) {
      if (m_ref == -INFINITY) m_ref = mx;  // first non-empty tile: nothing accumulated yet
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

    // ---- O^T += V^T . P^T ----
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int tile = 0; tile < 16; ++tile) {
        const uint32_t off = pv_off[tile & 1] + 16 * j * kRowLds + 128 * (tile >> 1);
        const half4 lo = lds_read_tr(buf, off);
        const half4 hi = lds_read_tr(buf, off + 8 * kRowLds);
        const half8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[tile] = mfma32x32x16(av, p[j], o[tile]);
      }
    }
  }
}

__global__ __launch_bounds__(256, 1) void decode_h128_bf16(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kBuf128];
  const ItemRange it = item_range(a);
  if (!it.ok) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hl = lane & 31;           // head within the wave / MFMA column
  const int g = lane >> 5;            // k-half of the MFMA operands
  const int h = wave * 32 + hl;

  // Q^T as the B operand: lane holds q_abs[b][h][16 ks + 8 g .. +7].
  half8 q[kDk / 16];
  {
    const uint16_t* qp = a.q_abs + ((int64_t)it.b * 128 + h) * kDk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kDk / 16; ++ks) q[ks] = __builtin_bit_cast(half8, ld16(qp + 16 * ks));
  }

  // Per-lane LDS offsets (swizzled chunks; see swz()).  Score operand: row hl,
  // chunk 2 ks + g.  Transposed value read: row 16 j + 4 g + (gi >> 2) (+8),
  // chunk 4 tile + 2 (grp & 1) + ((gi & 3) >> 1), 8 bytes in when gi is odd.
  const int grp = lane >> 4, gi = lane & 15;
  uint32_t qk_off[4];
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) qk_off[k4] = swz(hl, 2 * k4 + g);
  const int pv_row = 4 * g + (gi >> 2);
  uint32_t pv_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    pv_off[par] = swz(pv_row, 4 * par + 2 * (grp & 1) + ((gi & 3) >> 1)) + 8 * (gi & 1);

  floatx16 o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = floatx16{};
  float m_ref = -INFINITY, l_sum = 0.f;
  bool overflow = false;
  h128_pass<0>(a, it, lds, q, o, m_ref, l_sum, overflow, qk_off, pv_off);
  if (__syncthreads_or(overflow)) {
    // Rare: some head's scores grew by more than 2^kTauFixed after its first
    // tile.  Find the exact maxima, then redo the item against them.
    m_ref = -INFINITY;
    h128_pass<1>(a, it, lds, q, o, m_ref, l_sum, overflow, qk_off, pv_off);
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = floatx16{};
    l_sum = 0.f;
    h128_pass<2>(a, it, lds, q, o, m_ref, l_sum, overflow, qk_off, pv_off);
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

__global__ __launch_bounds__(256, 1) void decode_h16_bf16(DecodeArgs a) {
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

  LoaderBf16<kTile16> ld;
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
  for (int par = 0; par < 2; ++par) qk_off[par] = swz(tw + hl, 4 * par + grp);
  const int pv_row = tw + 4 * grp + (hl >> 2);
  uint32_t pv_off[4];
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4) pv_off[t4] = swz(pv_row, 2 * t4 + ((hl & 3) >> 1)) + 8 * (hl & 1);

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
hipError_t launch_decode_attn(const DecodeArgs& a, int num_heads, int cache_dtype, hipStream_t stream) {
  if (a.n_items <= 0) return hipSuccess;
  const dim3 grid(a.n_items), block(256);
  if (cache_dtype != 0) return hipErrorInvalidValue;
  if (num_heads == 128)
    hipLaunchKernelGGL(decode_h128_bf16, grid, block, 0, stream, a);
  else if (num_heads == 16)
    hipLaunchKernelGGL(decode_h16_bf16, grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mla
