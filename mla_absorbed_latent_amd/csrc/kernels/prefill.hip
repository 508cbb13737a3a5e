// prefill.hip -- chunked prefill attention in the unabsorbed form.
//
// Prefill is the compute-heavy side, where engines rebuild each head's key and
// value from the latent instead of folding W_UK into the query
// ("手搓 MLA:从 MHA 到 weight absorption,看懂 DeepSeek 的 KV 压缩" §四; the
// unabsorbed computation itself is that page's §三):
//   K_h[j] = [W_UK[h] c_j ; k_pe_j]   (128 + 64),   V_h[j] = W_UV[h] c_j   (128),
//   out[i][h] = softmax_j<=p_i(scale q_i,h . K_h[j]) V_h,   p_i = L - T + i.
// A chunk is the last T of L positions of one sequence; the first L - T are a
// prefix already in the cache, and query i attends to positions 0..p_i.
//
// Two kernels, both on the matrix cores (fp32 sums):
//   expand_kv_kernel: K_nope [H][Lp][128] and V^T [H][128][Lp] (fp16, Lp = L
//     rounded up to 64; pad positions repeat position L - 1, finite and always
//     masked) from c_kv and W_UK / W_UV, a tiled bf16 MFMA GEMM;
//   prefill_attn_kernel: flash attention per (128 queries, head): 4 waves of
//     32 queries, S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_f16
//     (each LDS fragment feeds two products), streaming softmax in fp32; a
//     work-group takes one query block, or two paired ones (a long and a
//     short causal range) when the whole grid fits the CUs at once.
// The operands of the attention products are fp16 (bf16 inputs widen exactly);
// P is rounded to fp16, its fp32 sum taken before rounding.
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

__device__ __forceinline__ floatx4 mfma16x16x32_bf16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two fp16 (round to nearest even), packed low | high.
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

// Grid (ceil(Lp / 256), H, 2); z = 0 writes K_nope, z = 1 writes V^T.  A
// work-group computes 256 positions x the 128 output features of head h as a
// tiled GEMM over the 512 latent channels, in 16 stages of 32 channels: a
// stage's latent rows and weight rows (64 B each) go straight into LDS, three
// stage buffers deep, so that two stages are in flight while one is used (72 KB
// of LDS: two work-groups fit a CU).  16-byte chunk c of row r sits at
// c ^ ((r >> 1) & 2).  A 16-byte LDS read serves 16 lanes per cycle, lanes
// 0-7 with 16-23 (and 8-15 with 24-31, and so on: the lanes whose bit 3 is
// equal), so that the 8 rows and two chunk columns (g, g ^ 1) of such a lane
// set must fill the 64 banks once: rows r and r + 4 share their banks and
// differ in bit 1 of the chunk (the swizzle c ^ ((r >> 2) & 3) made them
// collide, twice the cycles per fragment read; the prefill attention's
// layouts already met this).  Wave (wm, wn) computes 128 positions x
// 64 features (8 x 4 tiles of 16 x 16: 12 fragment reads feed 32 products;
// with 64 x 64 per wave, 8 fed 16).  Both operands are rows of channels
// with the same fragment layout, so the weight is the A operand for K_nope
// (D[feature][position]: four consecutive features per lane and store) and the
// B operand for V^T (D[position][feature]: four consecutive positions).
// V^T keeps each 32-key block's positions in the order 0-3, 16-19, 4-7, 20-23,
// 8-11, 24-27, 12-15, 28-31: the eight keys that lane group g of the value
// product takes in a k-step (32 ks + 4 g .. +3 and 32 ks + 16 + 4 g .. +3) are
// then one contiguous 16-byte chunk.  vt_pos maps a position j (a multiple of
// 4) to its stored place.
__device__ __forceinline__ int vt_pos(int j) {
  const int q = (j & 31) >> 2;
  return (j & ~31) + 4 * (q < 4 ? 2 * q : 2 * (q - 4) + 1);
}

constexpr int kXT = 256;                  // positions per work-group
constexpr int kXF = 128;                  // output features per work-group (one head's K_nope or V)
constexpr int kXChunk = 32;               // channels per stage
constexpr int kXRow = kXChunk * 2;        // 64 B
constexpr int kXBuf = (kXT + kXF) * kXRow;  // latent + weight rows of a stage, 24 KB
constexpr int kXStages = 3;               // stage buffers
constexpr int kXLoads = kXBuf / 1024 / 4; // 1 KB direct loads per wave per stage
constexpr int kXPT = kXT / 2 / 16;        // 16-position tiles per wave (8)
constexpr int kXFT = kXF / 2 / 16;        // 16-feature tiles per wave (4)

// s_waitcnt with only vmcnt constrained (gfx9 encoding).
template <int kN>
__device__ __forceinline__ void x_wait_vm() {
  __builtin_amdgcn_s_waitcnt((kN & 15) | (7 << 4) | (15 << 8) | ((kN >> 4) << 14));
}

template <bool is_v>
__device__ __forceinline__ void expand_kv_body(const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ w_in,
                                               int L, int Lp, uint16_t* __restrict__ k_nope,
                                               uint16_t* __restrict__ v_t, char* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;          // positions 128 wm.., features 64 wn..
  const int h = blockIdx.y;
  const int j0 = blockIdx.x * kXT;
  const uint16_t* w = w_in + (int64_t)h * kDn * kDc;

  // Staging: rows 0..255 latent, 256..383 weight, 4 chunks of 16 B per row,
  // straight into LDS (global_load_lds_dwordx4: lane i of a wave instruction
  // fills bytes 16 i .. of a 1 KB segment): 24 segments, wave w issues w + 4 i.
  // Each lane loads the chunk that belongs at its slot.  Positions past L load
  // position L - 1: finite values, masked in attention.
  const uint16_t* src0[kXLoads];
#pragma unroll
  for (int i = 0; i < kXLoads; ++i) {
    const int seg = wave + 4 * i, P = 64 * seg + lane, row = P >> 2, ch = (P & 3) ^ ((row >> 1) & 2);
    if (row < kXT) {
      const int j = j0 + row;
      src0[i] = c_kv + (int64_t)(j < L ? j : L - 1) * kDc + 8 * ch;
    } else {
      src0[i] = w + (int64_t)(row - kXT) * kDc + 8 * ch;
    }
  }
  auto issue = [&](int kc) {
    char* base = lds + (kc % kXStages) * kXBuf;
#pragma unroll
    for (int i = 0; i < kXLoads; ++i)
      __builtin_amdgcn_global_load_lds(src0[i] + kc * kXChunk,
                                       (__attribute__((address_space(3))) void*)(base + 1024 * (wave + 4 * i)), 16,
                                       0, 0);
  };

  floatx4 acc[kXPT][kXFT];
#pragma unroll
  for (int a = 0; a < kXPT; ++a)
#pragma unroll
    for (int b = 0; b < kXFT; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

  constexpr int kChunks = kDc / kXChunk;
  static_assert(kChunks >= kXStages, "the prologue fills kXStages - 1 stages");
#pragma unroll
  for (int kc = 0; kc < kXStages - 1; ++kc) issue(kc);
  // Stages fully unrolled, so that every wait count and buffer is a constant.
  // The barrier is a bare s_barrier after this wave's own waits: the workgroup
  // fence of __syncthreads would wait for every load in flight, the later
  // stages' included.
#pragma unroll
  for (int kc = 0; kc < kChunks; ++kc) {
    // stage kc's loads retire; the later stage (if any) stays in flight
    static_assert(kXStages == 3, "one later stage in flight at each wait");
    if (kc + 1 < kChunks) x_wait_vm<kXLoads>();
    else x_wait_vm<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // stage kc in LDS; stage kc - 1 read
    if (kc + kXStages - 1 < kChunks) issue(kc + kXStages - 1);
    const char* buf = lds + (kc % kXStages) * kXBuf;
    u32x4 wf[kXFT];
#pragma unroll
    for (int t = 0; t < kXFT; ++t) {
      const int wr = kXT + 64 * wn + 16 * t + li;
      wf[t] = *reinterpret_cast<const u32x4*>(buf + wr * kXRow + 16 * (g ^ ((wr >> 1) & 2)));
    }
    // Each position fragment feeds kXFT products.
#pragma unroll
    for (int a = 0; a < kXPT; ++a) {
      const int pr = 128 * wm + 16 * a + li;
      const u32x4 pf = *reinterpret_cast<const u32x4*>(buf + pr * kXRow + 16 * (g ^ ((pr >> 1) & 2)));
#pragma unroll
      for (int b = 0; b < kXFT; ++b) {
        // a: position tile, b: feature tile
        if constexpr (!is_v)
          acc[a][b] = mfma16x16x32_bf16(__builtin_bit_cast(bf16x8, wf[b]), __builtin_bit_cast(bf16x8, pf),
                                        acc[a][b]);
        else
          acc[a][b] = mfma16x16x32_bf16(__builtin_bit_cast(bf16x8, pf), __builtin_bit_cast(bf16x8, wf[b]),
                                        acc[a][b]);
      }
    }
  }

  // The fp16 result tile goes out through LDS as whole rows: for K_nope 256
  // position rows of 256 B, for V^T 128 feature rows of 512 B (positions in the
  // order of vt_pos).  Stored straight from the accumulators, each lane would
  // write 8-byte pieces of 16 different rows.  16-byte chunk c of tile row r
  // sits at c ^ (r & 15), so the 16 rows a store instruction touches hit
  // distinct banks.
  constexpr int kOutRow = is_v ? 2 * kXT : 2 * kXF;  // bytes per tile row
  static_assert(kXT * kXF * 2 <= kXStages * kXBuf, "the output tile fits in the stage buffers");
  __syncthreads();                                   // every wave is done with the stage buffers
  auto tile_off = [](int r, int col) {               // col: element (fp16) index within the row
    return r * kOutRow + 16 * ((col >> 3) ^ (r & 15)) + 2 * (col & 7);
  };
#pragma unroll
  for (int a = 0; a < kXPT; ++a)
#pragma unroll
    for (int b = 0; b < kXFT; ++b) {
      const u32x2 o = {pack_f16(acc[a][b][0], acc[a][b][1]), pack_f16(acc[a][b][2], acc[a][b][3])};
      if constexpr (!is_v) {
        // D[feature 64 wn + 16 b + 4 g + r][position 128 wm + 16 a + li]
        *reinterpret_cast<u32x2*>(lds + tile_off(128 * wm + 16 * a + li, 64 * wn + 16 * b + 4 * g)) = o;
      } else {
        // D[position 128 wm + 16 a + 4 g + r][feature 64 wn + 16 b + li]; the four
        // positions go to their place in the key order of vt_pos
        *reinterpret_cast<u32x2*>(lds + tile_off(64 * wn + 16 * b + li, vt_pos(128 * wm + 16 * a + 4 * g))) = o;
      }
    }
  __syncthreads();
  constexpr int kChunksPerRow = kOutRow / 16;        // 16 (K_nope) or 32 (V^T)
  constexpr int kRowsPerPass = 256 / kChunksPerRow;
#pragma unroll
  for (int pass = 0; pass < kXT * kXF * 2 / (256 * 16); ++pass) {
    const int r = kRowsPerPass * pass + tid / kChunksPerRow, c = tid % kChunksPerRow;
    const u32x4 v = *reinterpret_cast<const u32x4*>(lds + r * kOutRow + 16 * (c ^ (r & 15)));
    if constexpr (!is_v) {
      const int j = j0 + r;
      if (j < Lp) *reinterpret_cast<u32x4*>(k_nope + ((int64_t)h * Lp + j) * kDn + 8 * c) = v;
    } else {
      const int j = j0 + 8 * c;                      // positions j .. j + 7 in stored order
      if (j < Lp) *reinterpret_cast<u32x4*>(v_t + ((int64_t)h * kDn + r) * Lp + j) = v;
    }
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void expand_kv_kernel(const uint16_t* __restrict__ c_kv,
                                                        const uint16_t* __restrict__ w_uk,
                                                        const uint16_t* __restrict__ w_uv, int L, int Lp,
                                                        uint16_t* __restrict__ k_nope, uint16_t* __restrict__ v_t) {
  __shared__ __attribute__((aligned(16))) char lds[kXStages * kXBuf];
  if (blockIdx.z == 0) expand_kv_body<false>(c_kv, w_uk, L, Lp, k_nope, v_t, lds);
  else expand_kv_body<true>(c_kv, w_uv, L, Lp, k_nope, v_t, lds);
}

// Grid (ceil(T / kQB), H), kWaves waves.  Wave w owns queries
// i = kQB qb + 16 (kU w + u) + (lane % 16), u < kU; each K / V^T fragment read
// from LDS feeds kU products.  Per 64-key block: S^T[key][query] (4 key
// tiles x 6 k-steps), softmax per query column (its 64 keys sit in the four
// lanes l % 16 = q), then O^T[vdim][query] += V^T P^T (8 vdim tiles x 2
// k-steps).  P^T feeds the second product straight from the score registers:
// k index 8 g + e of a k-step stands for key 32 ks + 4 g + e (e < 4) or
// 32 ks + 16 + 4 g + e - 4, and V^T is read from LDS in the same order.
//
// Tiles go from global memory straight into LDS (global_load_lds_dwordx4: lane
// i of a wave instruction writes bytes 16 i .. 16 i + 15 of a 1 KB segment),
// double-buffered: the loads of block kb + 1 run under the products of block
// kb, and one barrier per block separates the two.  Each lane picks the global
// 16-byte chunk that belongs at its LDS slot, which gives the layouts
//   K tile   [64 keys][24 chunks of 8] (128 K_nope dims fp16, then 64 k_pe dims
//            kept in bf16), chunk c of key k at slot c ^ (k & 7);
//   V^T tile [128 dims][8 chunks of 8 keys] fp16 (keys in the order of vt_pos, so
//            chunk 4 ks + g is exactly the eight keys lane group g needs in
//            k-step ks), chunk c of dim d at c ^ (d & 7);
// the XOR spreads the 16 rows a fragment read touches over distinct banks.  The
// RoPE part of the scores uses the bf16 matrix instruction on the bf16 q_pe and
// k_pe (the products are exact either way).
constexpr int kWaves = 4;                 // waves per work-group
constexpr int kU = 2;                     // 16-query groups per wave
constexpr int kQB = 16 * kU * kWaves;     // queries per work-group
constexpr int kKSeg = 24 / kWaves;        // 1 KB K-tile segments per wave
constexpr int kVSeg = 16 / kWaves;        // 1 KB V^T-tile segments per wave
constexpr int kThreads = 64 * kWaves;
constexpr int kKBytes = 64 * 24 * 16;     // 24,576
constexpr int kVBytes = 128 * 8 * 16;     // 16,384
constexpr int kBufBytes = kKBytes + kVBytes;

typedef __attribute__((address_space(3))) void lds_void;

// One query block qb of head h (the work of one work-group; see the kernel).
__device__ __forceinline__ void prefill_qblock(const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
                                               const uint16_t* __restrict__ k_pe,
                                               const uint16_t* __restrict__ k_nope,
                                               const uint16_t* __restrict__ v_t, int T, int L, int Lp, int H,
                                               float scale_log2, uint16_t* __restrict__ out,
                                               float* __restrict__ lse, char* lds, int h, int qb) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int p_first = L - T + qb * kQB;
  const int p_last = L - T + min(qb * kQB + kQB - 1, T - 1);
  const int n_blocks = p_last / 64 + 1;

  int i_raw[kU], qpos[kU];
  u32x4 qf[kU][6];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    i_raw[u] = qb * kQB + 16 * (kU * wave + u) + li;
    const int i = i_raw[u] < T ? i_raw[u] : T - 1;   // rows past T repeat the last query, never stored
    qpos[u] = L - T + i;
    // Q^T fragments: dims 32 ks + 8 g .. +7 of query i (q_nope widened to fp16,
    // exact; q_pe stays bf16).
    const uint16_t* qn = q_nope + ((int64_t)i * H + h) * kDn + 8 * g;
    const uint16_t* qp = q_pe + ((int64_t)i * H + h) * kDr + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[u][ks] = bf16x8_to_f16x8(ld16(qn + 32 * ks));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qf[u][4 + ks] = ld16(qp + 32 * ks);
  }

  // This lane's part of a tile: K segments wave + 4 n (LDS slot P = 64 segment
  // + lane = 24 key + (chunk ^ (key & 7))), V^T segments wave + 4 n (P = 8 dim +
  // (chunk ^ (dim & 7))).  Each load's source for block 0 is formed here and
  // advanced by a fixed stride per block; pad keys (j >= L: only their k_pe
  // part, K_nope is padded) read row L - 1 instead.
  const uint16_t* k_nope_h = k_nope + (int64_t)h * Lp * kDn;
  const uint16_t* v_t_h = v_t + (int64_t)h * kDn * Lp;
  const char* ksrc[kKSeg];
  int kstride[kKSeg], kkey[kKSeg];
  const char* kpe_last[kKSeg];
#pragma unroll
  for (int n = 0; n < kKSeg; ++n) {
    const int P = 64 * (wave + kWaves * n) + lane, key = P / 24, ch = (P % 24) ^ (key & 7);
    kkey[n] = ch < 16 ? -1 : key;             // k_pe chunks check for pad keys
    ksrc[n] = ch < 16 ? reinterpret_cast<const char*>(k_nope_h + key * kDn + 8 * ch)
                      : reinterpret_cast<const char*>(k_pe + key * kDr + 8 * (ch - 16));
    kstride[n] = ch < 16 ? 64 * kDn * 2 : 64 * kDr * 2;
    kpe_last[n] = reinterpret_cast<const char*>(k_pe + (int64_t)(L - 1) * kDr + 8 * (ch < 16 ? 0 : ch - 16));
  }
  const char* vsrc[kVSeg];
#pragma unroll
  for (int n = 0; n < kVSeg; ++n) {
    const int P = 64 * (wave + kWaves * n) + lane, d = P >> 3, ch = (P & 7) ^ (d & 7);
    vsrc[n] = reinterpret_cast<const char*>(v_t_h + d * Lp + 8 * ch);
  }
  // Load m (0 .. kKSeg + kVSeg - 1) of block kb into buffer buf.
  auto issue_one = [&](int m, int kb, int buf) {
    char* base = lds + buf * kBufBytes;
    if (m < kKSeg) {
      const int n = m;
      const char* src = ksrc[n] + (int64_t)kb * kstride[n];
      if (kkey[n] >= 0 && kb * 64 + kkey[n] >= L) src = kpe_last[n];
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(base + 1024 * (wave + kWaves * n)), 16, 0, 0);
    } else {
      const int n = m - kKSeg;
      __builtin_amdgcn_global_load_lds(vsrc[n] + kb * 128, (lds_void*)(base + kKBytes + 1024 * (wave + kWaves * n)),
                                       16, 0, 0);
    }
  };
  auto issue = [&](int kb, int buf) {
#pragma unroll
    for (int m = 0; m < kKSeg + kVSeg; ++m) issue_one(m, kb, buf);
  };

  floatx4 o[kU][8];
  float m_run[kU], l_run[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[u][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    m_run[u] = -INFINITY;
    l_run[u] = 0.f;
  }

  issue(0, 0);
  for (int kb = 0; kb < n_blocks; ++kb) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();                                   // tile kb in LDS; block kb - 1 done by every wave
    // The last block re-loads itself into the idle buffer (never read) rather
    // than branching around the loads.
    const int kb_next = kb + 1 < n_blocks ? kb + 1 : kb;
    const char* kt_lds = lds + (kb & 1) * kBufBytes;
    const char* vt_lds = kt_lds + kKBytes;

    // Score products; the next block's loads are spread between them (one
    // after every other K fragment), so that the CU's load queue drains while
    // the matrix cores work instead of stalling every wave at the block start.
    // K fragment idx = 6 kt + ks (key tile kt, k-step ks) is read one step
    // ahead of its products.
    auto kfrag = [&](int idx) {
      const int kt = idx / 6, ks = idx % 6, key = 16 * kt + li;
      return *reinterpret_cast<const u32x4*>(kt_lds + key * 384 + 16 * ((4 * ks + g) ^ (key & 7)));
    };
    floatx4 s[kU][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int u = 0; u < kU; ++u) s[u][kt] = floatx4{0.f, 0.f, 0.f, 0.f};
    constexpr int kKPf = 3;                            // K fragments read ahead of their products
    u32x4 a_pf[kKPf];
#pragma unroll
    for (int d = 0; d < kKPf; ++d) a_pf[d] = kfrag(d);
#pragma unroll
    for (int idx = 0; idx < 24; ++idx) {
      const int kt = idx / 6, ks = idx % 6;
      const u32x4 a = a_pf[idx % kKPf];
      if (idx + kKPf < 24) a_pf[idx % kKPf] = kfrag(idx + kKPf);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (ks < 4)
          s[u][kt] = mfma16x16x32(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, qf[u][ks]), s[u][kt]);
        else
          s[u][kt] = mfma16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qf[u][ks]),
                                       s[u][kt]);
      }
      constexpr int kLoads = kKSeg + kVSeg;
      if ((idx & 1) && (idx >> 1) < kLoads) issue_one(idx >> 1, kb_next, (kb + 1) & 1);
    }
    // keys after the query (and pad keys) masked; only blocks that reach past
    // the work-group's first query can hold such keys
    if (kb * 64 + 63 > p_first) {
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kb * 64 + 16 * kt + 4 * g + r > qpos[u]) s[u][kt][r] = -INFINITY;
    }
    // streaming softmax on raw scores: p = 2^(c s - c m) with c = scale log2(e)
    u32x4 pb[kU][2];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float mb = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mb = fmaxf(mb, s[u][kt][r]);
      mb = max_xor16_32(mb);
      const float m_new = fmaxf(m_run[u], mb);       // finite: key 0 is in every query's range
      const float alpha = __builtin_amdgcn_exp2f((m_run[u] - m_new) * scale_log2);
      m_run[u] = m_new;
      const float neg_mc = -m_new * scale_log2;
      float lsum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[u][kt][r], scale_log2, neg_mc));
          s[u][kt][r] = p;
          lsum += p;
        }
      l_run[u] = l_run[u] * alpha + lsum;
      // the running maximum of most columns stops moving after a few blocks:
      // rescale only when some column's changed (alpha == 1 leaves o as it is)
      if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) o[u][mt] *= alpha;
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        pb[u][ks] = u32x4{pack_f16(s[u][2 * ks][0], s[u][2 * ks][1]), pack_f16(s[u][2 * ks][2], s[u][2 * ks][3]),
                          pack_f16(s[u][2 * ks + 1][0], s[u][2 * ks + 1][1]),
                          pack_f16(s[u][2 * ks + 1][2], s[u][2 * ks + 1][3])};
    }
    // V^T fragment idx = 8 ks + mt, read kVPf products ahead.
    constexpr int kVPf = 2;
    auto vfrag = [&](int idx) {
      const int ks = idx / 8, d = 16 * (idx % 8) + li;
      return *reinterpret_cast<const u32x4*>(vt_lds + d * 128 + 16 * ((4 * ks + g) ^ (d & 7)));
    };
    u32x4 v_pf[kVPf];
#pragma unroll
    for (int d = 0; d < kVPf; ++d) v_pf[d] = vfrag(d);
#pragma unroll
    for (int idx = 0; idx < 16; ++idx) {
      const int ks = idx / 8, mt = idx % 8;
      const half8 av = __builtin_bit_cast(half8, v_pf[idx % kVPf]);
      if (idx + kVPf < 16) v_pf[idx % kVPf] = vfrag(idx + kVPf);
#pragma unroll
      for (int u = 0; u < kU; ++u) o[u][mt] = mfma16x16x32(av, __builtin_bit_cast(half8, pb[u][ks]), o[u][mt]);
    }
  }

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the last block's idle re-load has landed
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    float l = l_run[u];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (i_raw[u] < T) {
      const float inv = 1.f / l;
      uint16_t* orow = out + ((int64_t)i_raw[u] * H + h) * kDn + 4 * g;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const uint32_t a = (uint32_t)f32_to_bf16_rne(o[u][mt][0] * inv) | ((uint32_t)f32_to_bf16_rne(o[u][mt][1] * inv) << 16);
        const uint32_t b = (uint32_t)f32_to_bf16_rne(o[u][mt][2] * inv) | ((uint32_t)f32_to_bf16_rne(o[u][mt][3] * inv) << 16);
        *reinterpret_cast<u32x2*>(orow + 16 * mt) = u32x2{a, b};
      }
      if (lse != nullptr && g == 0)
        lse[(int64_t)i_raw[u] * H + h] = (m_run[u] * scale_log2 + __log2f(l)) * 0.6931471805599453f;
    }
  }
}

// Work-groups are dealt to the 8 XCDs round robin by linear id.  With H a
// multiple of 8 (16 or 128), the k-th work-group of XCD x takes head
// x + 8 (k / units) and unit k % units of it: all query blocks of a head run
// on one XCD (its K/V stays in that L2).  Unit u is query block nqb - 1 - u
// (longest causal ranges first), or, with kPairs (nqb even), query blocks
// nqb - 1 - u and then u: every work-group then has the same number of key
// blocks.  Pairs serve launches whose work-groups all fit the CUs at once
// (16-head prompts), where the longest causal range would otherwise set the
// time while the CUs of the short ones idle.
template <bool kPairs>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_attn_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe, const uint16_t* __restrict__ k_pe,
    const uint16_t* __restrict__ k_nope, const uint16_t* __restrict__ v_t, int T, int L, int Lp, int H,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * kBufBytes];
  const int units = gridDim.x;
  const int nqb = kPairs ? 2 * units : units;
  const int wg_id = blockIdx.x + units * blockIdx.y;
  const int xcd = wg_id & 7, k_on_xcd = wg_id >> 3;
  const int h = xcd + 8 * (k_on_xcd / units);
  const int unit = k_on_xcd % units;
  prefill_qblock(q_nope, q_pe, k_pe, k_nope, v_t, T, L, Lp, H, scale_log2, out, lse, lds, h, nqb - 1 - unit);
  if constexpr (kPairs) {
    __syncthreads();                       // every wave is done with the first block's tiles
    prefill_qblock(q_nope, q_pe, k_pe, k_nope, v_t, T, L, Lp, H, scale_log2, out, lse, lds, h, unit);
  }
}

}  // namespace

constexpr int kNumCUs = 256;             // compute units of a gfx950 card (8 XCDs x 32)

int64_t prefill_padded_len(int seq_len) { return ((int64_t)seq_len + 63) / 64 * 64; }

hipError_t launch_prefill_attn(int num_heads, float softmax_scale, const uint16_t* q_nope, const uint16_t* q_pe,
                               int n_queries, const uint16_t* c_kv, const uint16_t* k_pe, int seq_len,
                               const uint16_t* w_uk, const uint16_t* w_uv, void* workspace, uint16_t* out,
                               float* lse, hipStream_t stream) {
  if (n_queries <= 0) return hipSuccess;
  const int64_t Lp = prefill_padded_len(seq_len);
  uint16_t* k_nope = static_cast<uint16_t*>(workspace);
  uint16_t* v_t = k_nope + (int64_t)num_heads * Lp * kDn;
  hipLaunchKernelGGL(expand_kv_kernel, dim3((unsigned)((Lp + kXT - 1) / kXT), num_heads, 2), dim3(256), 0, stream,
                     c_kv, w_uk,
                     w_uv, seq_len, (int)Lp, k_nope, v_t);
  // Pair the query blocks when the whole grid fits the CUs at once (two
  // work-groups per CU): a CU then holds one long and one short causal range.
  const int nqb = (n_queries + kQB - 1) / kQB;
  const bool pairs = nqb % 2 == 0 && (int64_t)nqb * num_heads <= 2 * kNumCUs;
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  if (pairs)
    hipLaunchKernelGGL(prefill_attn_kernel<true>, dim3(nqb / 2, num_heads), dim3(kThreads), 0, stream, q_nope, q_pe,
                       k_pe, k_nope, v_t, n_queries, seq_len, (int)Lp, num_heads, scale_log2, out, lse);
  else
    hipLaunchKernelGGL(prefill_attn_kernel<false>, dim3(nqb, num_heads), dim3(kThreads), 0, stream, q_nope, q_pe,
                       k_pe, k_nope, v_t, n_queries, seq_len, (int)Lp, num_heads, scale_log2, out, lse);
  return hipGetLastError();
}

}  // namespace mla
