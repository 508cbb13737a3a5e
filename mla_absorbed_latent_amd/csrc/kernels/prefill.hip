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
//     rounded up to 64, pad positions zero) from c_kv and W_UK / W_UV (bf16 MFMA);
//   prefill_attn_kernel: flash attention per (64 queries, head), S^T = K Q^T and
//     O^T = V^T P^T on v_mfma_f32_16x16x32_f16, streaming softmax in fp32.
// The operands of the attention products are fp16 (bf16 inputs widen exactly);
// P is rounded to fp16, its fp32 sum taken before rounding.
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int kKRow = 192 * 2 + 16;   // LDS bytes per key row (K_nope | k_pe, fp16) + 16 B pad
constexpr int kVRow = 64 * 2 + 8;     // LDS bytes per V^T row (64 keys, fp16) + 8 B pad
constexpr int kKTile = 64 * kKRow;    // 25,600 B
constexpr int kVTile = 128 * kVRow;   // 17,408 B

__device__ __forceinline__ floatx4 mfma16x16x32_bf16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return (uint32_t)f32_to_f16_bits(a) | ((uint32_t)f32_to_f16_bits(b) << 16);
}

// Grid (Lp / 64, H, 2); z = 0 writes K_nope, z = 1 writes V^T.  Wave w covers
// positions 64 bx + 16 w .. +15; its latent fragments (512 channels, the same
// register layout serves as A or B) stay in registers while it walks the 128
// output features of head h in tiles of 16.
__global__ __launch_bounds__(256) void expand_kv_kernel(const uint16_t* __restrict__ c_kv,
                                                        const uint16_t* __restrict__ w_uk,
                                                        const uint16_t* __restrict__ w_uv, int L, int Lp,
                                                        uint16_t* __restrict__ k_nope, uint16_t* __restrict__ v_t) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.y, is_v = blockIdx.z;
  const int g = lane >> 4, li = lane & 15;
  const int j0 = blockIdx.x * 64 + wave * 16;
  const int j = j0 + li;
  u32x4 cf[kDc / 32];
#pragma unroll
  for (int ks = 0; ks < kDc / 32; ++ks)
    cf[ks] = j < L ? ld16(c_kv + (int64_t)j * kDc + 32 * ks + 8 * g) : u32x4{0, 0, 0, 0};
  const uint16_t* w = (is_v ? w_uv : w_uk) + (int64_t)h * kDn * kDc;
  for (int mt = 0; mt < kDn / 16; ++mt) {
    const uint16_t* wr = w + (int64_t)(16 * mt + li) * kDc + 8 * g;
    u32x4 wf[kDc / 32];
#pragma unroll
    for (int ks = 0; ks < kDc / 32; ++ks) wf[ks] = ld16(wr + 32 * ks);
    floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
    if (!is_v) {
      // D[feature 16 mt + 4 g + r][position j0 + li]
#pragma unroll
      for (int ks = 0; ks < kDc / 32; ++ks)
        acc = mfma16x16x32_bf16(__builtin_bit_cast(bf16x8, wf[ks]), __builtin_bit_cast(bf16x8, cf[ks]), acc);
      u32x2 o = {pack_f16(acc[0], acc[1]), pack_f16(acc[2], acc[3])};
      *reinterpret_cast<u32x2*>(k_nope + ((int64_t)h * Lp + j) * kDn + 16 * mt + 4 * g) = o;
    } else {
      // D[position j0 + 4 g + r][feature 16 mt + li]
#pragma unroll
      for (int ks = 0; ks < kDc / 32; ++ks)
        acc = mfma16x16x32_bf16(__builtin_bit_cast(bf16x8, cf[ks]), __builtin_bit_cast(bf16x8, wf[ks]), acc);
      u32x2 o = {pack_f16(acc[0], acc[1]), pack_f16(acc[2], acc[3])};
      *reinterpret_cast<u32x2*>(v_t + ((int64_t)h * kDn + 16 * mt + li) * Lp + j0 + 4 * g) = o;
    }
  }
}

// Grid (ceil(T / 64), H), 256 threads; the query blocks run last-first (the
// longest causal ranges start first).  Wave w owns queries i = 64 qb + 16 w +
// (lane % 16).  Per 64-key block: S^T[key][query] (4 key tiles x 6 k-steps),
// softmax per query column (its 64 keys sit in the four lanes l % 16 = q),
// then O^T[vdim][query] += V^T P^T (8 vdim tiles x 2 k-steps).  P^T feeds the
// second product straight from the score registers: k index 8 g + e of a
// k-step stands for key 32 ks + 4 g + e (e < 4) or 32 ks + 16 + 4 g + e - 4,
// and V^T is read from LDS in the same order.
__global__ __launch_bounds__(256) void prefill_attn_kernel(const uint16_t* __restrict__ q_nope,
                                                           const uint16_t* __restrict__ q_pe,
                                                           const uint16_t* __restrict__ k_pe,
                                                           const uint16_t* __restrict__ k_nope,
                                                           const uint16_t* __restrict__ v_t, int T, int L, int Lp,
                                                           int H, float scale_log2, uint16_t* __restrict__ out,
                                                           float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) char k_lds[kKTile];
  __shared__ __attribute__((aligned(16))) char v_lds[kVTile];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int h = blockIdx.y;
  const int qb = gridDim.x - 1 - blockIdx.x;
  const int i_raw = qb * 64 + wave * 16 + li;
  const int i = i_raw < T ? i_raw : T - 1;         // rows past T repeat the last query, never stored
  const int qpos = L - T + i;
  const int p_first = L - T + qb * 64;
  const int p_last = L - T + min(qb * 64 + 63, T - 1);
  const int n_blocks = p_last / 64 + 1;

  // Q^T fragments: dims 32 ks + 8 g .. +7 of query i (bf16 -> fp16, exact).
  u32x4 qf[6];
  {
    const uint16_t* qn = q_nope + ((int64_t)i * H + h) * kDn + 8 * g;
    const uint16_t* qp = q_pe + ((int64_t)i * H + h) * kDr + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = bf16x8_to_f16x8(ld16(qn + 32 * ks));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) qf[4 + ks] = bf16x8_to_f16x8(ld16(qp + 32 * ks));
  }

  // Tile staging: 64 keys x 24 chunks of K (16 from K_nope, 8 from k_pe), and
  // 128 V^T rows x 8 chunks; six and four 16-byte loads per thread.
  u32x4 kr[6], vr[4];
  auto load_tile = [&](int kb) {
#pragma unroll
    for (int n = 0; n < 6; ++n) {
      const int idx = tid + 256 * n, key = idx / 24, ch = idx % 24;
      const int j = kb * 64 + key;
      if (ch < 16) {
        kr[n] = ld16(k_nope + ((int64_t)h * Lp + j) * kDn + 8 * ch);
      } else {
        const int jc = j < L ? j : L - 1;          // pad keys are masked; read a real row
        kr[n] = bf16x8_to_f16x8(ld16(k_pe + (int64_t)jc * kDr + 8 * (ch - 16)));
      }
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int idx = tid + 256 * n, d = idx >> 3, ch = idx & 7;
      vr[n] = ld16(v_t + ((int64_t)h * kDn + d) * Lp + kb * 64 + 8 * ch);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int n = 0; n < 6; ++n) {
      const int idx = tid + 256 * n, key = idx / 24, ch = idx % 24;
      *reinterpret_cast<u32x4*>(k_lds + key * kKRow + 16 * ch) = kr[n];
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int idx = tid + 256 * n, d = idx >> 3, ch = idx & 7;
      *reinterpret_cast<u32x2*>(v_lds + d * kVRow + 16 * ch) = u32x2{vr[n][0], vr[n][1]};
      *reinterpret_cast<u32x2*>(v_lds + d * kVRow + 16 * ch + 8) = u32x2{vr[n][2], vr[n][3]};
    }
  };

  floatx4 o[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) o[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  load_tile(0);
  for (int kb = 0; kb < n_blocks; ++kb) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kb + 1 < n_blocks) load_tile(kb + 1);

    floatx4 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
      const char* krow = k_lds + (16 * kt + li) * kKRow + 16 * g;
#pragma unroll
      for (int ks = 0; ks < 6; ++ks) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(krow + 64 * ks);
        s[kt] = mfma16x16x32(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, qf[ks]), s[kt]);
      }
    }
    // scores in log2 units; keys after the query (and pad keys) masked
    const bool diag = kb * 64 + 63 > p_first;
    float mb = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = s[kt][r] * scale_log2;
        if (diag && kb * 64 + 16 * kt + 4 * g + r > qpos) v = -INFINITY;
        s[kt][r] = v;
        mb = fmaxf(mb, v);
      }
    mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
    mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
    const float m_new = fmaxf(m_run, mb);            // finite: key 0 is in every query's range
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(s[kt][r] - m_new);
        s[kt][r] = p;
        lsum += p;
      }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] *= alpha;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 pb = {pack_f16(s[2 * ks][0], s[2 * ks][1]), pack_f16(s[2 * ks][2], s[2 * ks][3]),
                        pack_f16(s[2 * ks + 1][0], s[2 * ks + 1][1]), pack_f16(s[2 * ks + 1][2], s[2 * ks + 1][3])};
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const char* vrow = v_lds + (16 * mt + li) * kVRow + 2 * (32 * ks + 4 * g);
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 32);
        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
        o[mt] = mfma16x16x32(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, pb), o[mt]);
      }
    }
  }

  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (i_raw < T) {
    const float inv = 1.f / l_run;
    uint16_t* orow = out + ((int64_t)i * H + h) * kDn + 4 * g;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const uint32_t a = (uint32_t)f32_to_bf16_rne(o[mt][0] * inv) | ((uint32_t)f32_to_bf16_rne(o[mt][1] * inv) << 16);
      const uint32_t b = (uint32_t)f32_to_bf16_rne(o[mt][2] * inv) | ((uint32_t)f32_to_bf16_rne(o[mt][3] * inv) << 16);
      *reinterpret_cast<u32x2*>(orow + 16 * mt) = u32x2{a, b};
    }
    if (lse != nullptr && g == 0) lse[(int64_t)i * H + h] = (m_run + log2f(l_run)) * 0.6931471805599453f;
  }
}

}  // namespace

int64_t prefill_padded_len(int seq_len) { return ((int64_t)seq_len + 63) / 64 * 64; }

hipError_t launch_prefill_attn(int num_heads, float softmax_scale, const uint16_t* q_nope, const uint16_t* q_pe,
                               int n_queries, const uint16_t* c_kv, const uint16_t* k_pe, int seq_len,
                               const uint16_t* w_uk, const uint16_t* w_uv, void* workspace, uint16_t* out,
                               float* lse, hipStream_t stream) {
  if (n_queries <= 0) return hipSuccess;
  const int64_t Lp = prefill_padded_len(seq_len);
  uint16_t* k_nope = static_cast<uint16_t*>(workspace);
  uint16_t* v_t = k_nope + (int64_t)num_heads * Lp * kDn;
  hipLaunchKernelGGL(expand_kv_kernel, dim3((unsigned)(Lp / 64), num_heads, 2), dim3(256), 0, stream, c_kv, w_uk,
                     w_uv, seq_len, (int)Lp, k_nope, v_t);
  hipLaunchKernelGGL(prefill_attn_kernel, dim3((n_queries + 63) / 64, num_heads), dim3(256), 0, stream, q_nope,
                     q_pe, k_pe, k_nope, v_t, n_queries, seq_len, (int)Lp, num_heads,
                     softmax_scale * 1.4426950408889634f, out, lse);
  return hipGetLastError();
}

}  // namespace mla
