// combine_out.hip -- log-sum-exp merge of split-KV partials, and the output
// projections.
//
// Merge (one work-group per (sequence, head); exact for any split of the tokens):
//     lse = ln sum_j e^{lse_j},  o_lat = sum_j e^{lse_j - lse} o_j
// with the fp16 partials o_j widened and summed in fp32.
// An all-empty sequence gives o_lat = 0, lse = -inf; one split is a copy.
//
// Output projection ("DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界" §2.3:
// sum_t p_t W^V c_t = W^V sum_t p_t c_t; "手搓 MLA:从 MHA 到 weight absorption" §四,
// einsum "thc,hdc->thd"):
//     out[b,h,d] = sum_c W_UV[h,d,c] o_lat[b,h,c]
// run as out^T[d][b] = W_UV[h][d][c] . o_lat^T[c][b] on the fp16 matrix cores
// (mfma 32x32x16): both operands come straight from HBM with 16-byte loads,
// since each lane needs 8 consecutive c -- the contiguous axis of both W_UV and
// o_lat.  W_UV is widened bf16 -> fp16 exactly; o_lat is rounded fp32 -> fp16.
// The fp32 sums go to `out` as bf16 and, when a layer output is wanted, to an
// fp32 workspace for the W_O product.
//
// W_O product (optional): y[b,n] = sum_k W_O[n,k] x[b,k], x = concat_h out[b,h,:]
// in fp32; one wave per output feature, fp32 FMAs, a wave reduction.
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

__global__ __launch_bounds__(128) void combine_kernel(const uint16_t* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      const int32_t* __restrict__ offsets, float* __restrict__ o_lat,
                                                      float* __restrict__ lse_out, int H) {
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int r0 = offsets[b], r1 = offsets[b + 1];
  // The maximum in batches of eight independent loads.
  float m = -INFINITY;
  for (int j = r0; j < r1; j += 8) {
    float lb[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float lv = lse_part[(int64_t)min(j + k, r1 - 1) * H + h];
      lb[k] = j + k < r1 ? lv : -INFINITY;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, lb[k]);
  }
  floatx4 acc = floatx4{};
  float wsum = 0.f;
  if (m != -INFINITY) {
    // Four splits per round, in order: a round's rows are loaded while the round
    // before is weighted; an empty split (lse = -inf) contributes nothing,
    // whatever its row holds.
    auto load = [&](int j0, floatx4 (&x)[4], float (&l)[4]) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int j = min(j0 + k, r1 - 1);
        l[k] = j0 + k < r1 ? lse_part[(int64_t)j * H + h] : -INFINITY;
        x[k] = __builtin_convertvector(*reinterpret_cast<const half4*>(o_part + ((int64_t)j * H + h) * kDc + 4 * threadIdx.x),
                                      floatx4);
      }
    };
    floatx4 x[4];
    float l[4];
    load(r0, x, l);
    for (int j0 = r0; j0 < r1; j0 += 4) {
      floatx4 xn[4];
      float ln[4];
      load(j0 + 4, xn, ln);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bool empty = l[k] == -INFINITY;      // skipped outright, as if not loaded
        const float w = empty ? 0.f : expf(l[k] - m);
        wsum += w;
        acc += w * (empty ? floatx4{} : x[k]);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[k] = xn[k];
        l[k] = ln[k];
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  *reinterpret_cast<floatx4*>(o_lat + ((int64_t)b * H + h) * kDc + 4 * threadIdx.x) = acc * inv;
  if (lse_out != nullptr && threadIdx.x == 0) lse_out[(int64_t)b * H + h] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
}

// One work-group per (head, 32 rows of d).  Its four waves split c into
// quarters: each loads its W_UV slice and o_lat fragments up front (all
// independent 16-byte loads, so the memory system sees them at once), runs 16
// MFMAs per 64 sequences, and the four partial sums meet in LDS.
__global__ __launch_bounds__(256, 2) void out_proj_kernel(const float* __restrict__ o_lat,
                                                          const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ out,
                                                          float* __restrict__ out_f32, int H, int B) {
  __shared__ float red[4][2][16][64];              // [wave][b block][acc register][lane], 32 KB
  const int h = blockIdx.x >> 2;
  const int d0 = (blockIdx.x & 3) * 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5;
  const int cq = 128 * wave;                        // this wave's quarter of c

  // A operand: W_UV[h][d0 + lane % 32][cq + 16 ks + 8 g .. +7], widened exactly.
  u32x4 wr[8];
  const uint16_t* wrow = w_uv + ((int64_t)h * kDn + d0 + (lane & 31)) * kDc + cq + 8 * g;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) wr[ks] = ld16(wrow + 16 * ks);

  for (int b0 = 0; b0 < B; b0 += 64) {
    // B operand: o_lat[b][h][cq + 16 ks + 8 g .. +7], b = b0 + 32 bb + lane % 32.  All
    // loads of the chunk are issued before any is used.  A sequence past B reads
    // row 0 instead; its column of the product is never stored.
    floatx4 x[2][16];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int b = b0 + 32 * bb + (lane & 31);
      const float* orow = o_lat + ((int64_t)(b < B ? b : 0) * H + h) * kDc + cq + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        x[bb][2 * ks] = *reinterpret_cast<const floatx4*>(orow + 16 * ks);
        x[bb][2 * ks + 1] = *reinterpret_cast<const floatx4*>(orow + 16 * ks + 4);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    floatx16 acc[2] = {floatx16{}, floatx16{}};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const half8 a = __builtin_bit_cast(half8, bf16x8_to_f16x8(wr[ks]));
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const half4 lo = __builtin_convertvector(x[bb][2 * ks], half4);      // round to nearest even
        const half4 hi = __builtin_convertvector(x[bb][2 * ks + 1], half4);
        acc[bb] = mfma32x32x16(a, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), acc[bb]);
      }
    }
    __syncthreads();                               // the previous chunk's sums have been read
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[wave][bb][r][lane] = acc[bb][r];
    __syncthreads();
    // Thread t sums registers 8 rh .. 8 rh + 7 of lane l2 in b block bb over the four waves:
    // out^T[d0 + 8 (r / 4) + 4 (l2 / 32) + r % 4][b0 + 32 bb + l2 % 32].
    const int bb = threadIdx.x >> 7, rh = (threadIdx.x >> 6) & 1, l2 = threadIdx.x & 63;   // bank = l2: conflict free
    const int b = b0 + 32 * bb + (l2 & 31);
    if (b < B) {
#pragma unroll
      for (int q4 = 0; q4 < 2; ++q4) {
        floatx4 v = floatx4{};
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += red[w][bb][8 * rh + 4 * q4 + e][l2];
        const int d = d0 + 8 * (2 * rh + q4) + 4 * (l2 >> 5);
        u32x2 o2;
        o2[0] = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
        o2[1] = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
        *reinterpret_cast<u32x2*>(out + ((int64_t)b * H + h) * kDn + d) = o2;
        if (out_f32 != nullptr) *reinterpret_cast<floatx4*>(out_f32 + ((int64_t)b * H + h) * kDn + d) = v;
      }
    }
  }
}

// Merge and expansion in one pass, one work-group (8 waves) per (head, 32 sequences):
//  1. merge: the work-group combines, for each of its sequences, the fp16
//     partials of head h (fp32 sums, as combine_kernel), keeps o_lat[b][h][:]
//     as fp16 in LDS, and writes o_lat / lse as well when asked;
//  2. expand: wave w computes out^T[16 w .. 16 w + 15][b] = W_UV[h][d][:] . o_lat^T
//     for the 32 sequences (32 x mfma 16x16x32), W_UV rows from HBM and o_lat^T
//     fragments from LDS.
// Every load that does not depend on another is issued before the first use:
// the W_UV rows at entry, the split rows of all four of a thread's sequences
// together, so the kernel waits for about two memory round trips in all.  o_lat
// never leaves the chip, and one launch replaces two.
// Shapes with few (head, 32-sequence) groups (16 heads, a few dozen sequences)
// take work-groups of 8 sequences and a quarter of d each (each quarter merges
// its sequences again; the partials are small), so that enough CUs work.
constexpr int kCoThreads = 512;

template <int kCoB, int kCoRound, int kDSplit>
__global__ __launch_bounds__(kCoThreads, 1) void combine_out_proj_kernel(
    const uint16_t* __restrict__ o_part, const float* __restrict__ lse_part, const int32_t* __restrict__ offsets,
    const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ out, float* __restrict__ out_f32,
    float* __restrict__ o_lat, float* __restrict__ lse_out, int H, int B) {
  constexpr int kCoSeq = kCoB / (kCoThreads / 64);   // sequences per thread in the merge
  constexpr int kRows = kCoB < 16 ? 16 : kCoB;        // LDS rows (the MFMA takes 16 sequences)
  constexpr int kDPart = kDn / kDSplit;               // output rows d of this work-group
  constexpr int kWaves = kDPart / 16;                 // waves with expansion work
  static_assert(kCoSeq >= 1 && kRows % 16 == 0 && kWaves >= 1, "work-group shape");
  // o_lat tile, fp16: row bi (1 KB) holds sequence b0 + bi, 16-byte chunk c at
  // c ^ (bi & 15), so that the 16 rows a lane group reads land in distinct banks.
  __shared__ __attribute__((aligned(16))) char olds[kRows * kDc * 2];
  const int n_bc = (B + kCoB - 1) / kCoB;
  const int h = blockIdx.x % H;
  const int b0 = ((blockIdx.x / H) % n_bc) * kCoB;
  const int d0 = (blockIdx.x / (H * n_bc)) * kDPart;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // Sequence group of the merge: one per wave, made wave-uniform so that the
  // split offsets below come through scalar loads (a vector load of them,
  // queued behind the W_UV loads, made the split rows wait for W_UV).
  const int grp = __builtin_amdgcn_readfirstlane(t >> 6);

  // A operand of the expansion: W_UV[h][d0 + 16 wave + lane % 16][32 ks + 8 (lane / 16) .. +7].
  u32x4 wr[16];
  if (wave < kWaves) {
    const uint16_t* wrow = w_uv + ((int64_t)h * kDn + d0 + 16 * wave + (lane & 15)) * kDc + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) wr[ks] = ld16(wrow + 32 * ks);
  }

  // ---- 1. merge: thread t owns 16-byte chunk c8 = t % 64 of sequences b0 + grp + 8 i
  const int c8 = t & 63;
  int r0[kCoSeq], r1[kCoSeq];
#pragma unroll
  for (int i = 0; i < kCoSeq; ++i) {
    const int b = b0 + grp + 8 * i;
    r0[i] = b < B ? offsets[b] : 0;
    r1[i] = b < B ? offsets[b + 1] : 0;
  }
  // Every split row is loaded without a branch, from an index clamped into the
  // sequence's rows (row 0 for an empty one), and masked afterwards: a load
  // under a branch left its value to be copied at the join, and each copy
  // waited for its load.  With no split row at all (every sequence empty) the
  // loads read W_UV instead, which is always there; their values are masked.
  const bool any_rows = offsets[B] > 0;
  const uint16_t* op = any_rows ? o_part : w_uv;
  const float* lp = any_rows ? lse_part : reinterpret_cast<const float*>(w_uv);
  auto row_of = [&](int j, int i) { return max(min(j, r1[i] - 1), 0); };
  float l[kCoSeq][kCoRound];
  half8 x[kCoSeq][kCoRound];
#pragma unroll
  for (int i = 0; i < kCoSeq; ++i)
#pragma unroll
    for (int k = 0; k < kCoRound; ++k) {
      const int j = r0[i] + k, jc = row_of(j, i);
      const float lv = lp[(int64_t)jc * H + h];
      x[i][k] = *reinterpret_cast<const half8*>(op + ((int64_t)jc * H + h) * kDc + 8 * c8);
      l[i][k] = j < r1[i] ? lv : -INFINITY;
    }
#pragma unroll
  for (int i = 0; i < kCoSeq; ++i) {
    const int bi = grp + 8 * i, b = b0 + bi;
    // The same sums in the same order as combine_kernel: the maximum over all
    // rows first, then the rows in rounds of kCoRound; an empty split (lse =
    // -inf) contributes nothing, whatever its row holds.
    float m = -INFINITY, wsum = 0.f;
#pragma unroll
    for (int k = 0; k < kCoRound; ++k) m = fmaxf(m, l[i][k]);
    // The rest of the maximum in batches of eight independent loads (a long
    // sequence of a ragged batch has dozens of splits).
    for (int j = r0[i] + kCoRound; j < r1[i]; j += 8) {
      float lb[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float lv = lp[(int64_t)row_of(j + k, i) * H + h];
        lb[k] = j + k < r1[i] ? lv : -INFINITY;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) m = fmaxf(m, lb[k]);
    }
    floatx4 acc0 = floatx4{}, acc1 = floatx4{};
    if (m != -INFINITY) {
      // Rounds of kCoRound splits in order; each round's rows are loaded while
      // the round before is summed.
      float lr[kCoRound];
      half8 xr[kCoRound];
#pragma unroll
      for (int k = 0; k < kCoRound; ++k) {
        lr[k] = l[i][k];
        xr[k] = x[i][k];
      }
      for (int j0 = r0[i]; j0 < r1[i]; j0 += kCoRound) {
        float ln[kCoRound];
        half8 xn[kCoRound];
#pragma unroll
        for (int k = 0; k < kCoRound; ++k) {
          const int j = j0 + kCoRound + k, jc = row_of(j, i);
          const float lv = lp[(int64_t)jc * H + h];
          xn[k] = *reinterpret_cast<const half8*>(op + ((int64_t)jc * H + h) * kDc + 8 * c8);
          ln[k] = j < r1[i] ? lv : -INFINITY;
        }
#pragma unroll
        for (int k = 0; k < kCoRound; ++k) {
          const bool empty = lr[k] == -INFINITY;
          const float w = empty ? 0.f : expf(lr[k] - m);
          wsum += w;
          const floatx4 lo = __builtin_convertvector(__builtin_shufflevector(xr[k], xr[k], 0, 1, 2, 3), floatx4);
          const floatx4 hi = __builtin_convertvector(__builtin_shufflevector(xr[k], xr[k], 4, 5, 6, 7), floatx4);
          acc0 += w * (empty ? floatx4{} : lo);
          acc1 += w * (empty ? floatx4{} : hi);
        }
#pragma unroll
        for (int k = 0; k < kCoRound; ++k) {
          lr[k] = ln[k];
          xr[k] = xn[k];
        }
      }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    acc0 *= inv;
    acc1 *= inv;
    const half4 lo = __builtin_convertvector(acc0, half4), hi = __builtin_convertvector(acc1, half4);   // nearest even
    *reinterpret_cast<half8*>(olds + bi * (kDc * 2) + 16 * (c8 ^ (bi & 15))) =
        __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    if (b < B && d0 == 0) {
      if (o_lat != nullptr) {
        float* dst = o_lat + ((int64_t)b * H + h) * kDc + 8 * c8;
        *reinterpret_cast<floatx4*>(dst) = acc0;
        *reinterpret_cast<floatx4*>(dst + 4) = acc1;
      }
      if (lse_out != nullptr && c8 == 0) lse_out[(int64_t)b * H + h] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
    }
  }
  for (int bi = kCoB + grp; bi < kRows; bi += kCoThreads / 64)      // rows past kCoB: zeros
    *reinterpret_cast<half8*>(olds + bi * (kDc * 2) + 16 * (c8 ^ (bi & 15))) = half8{};
  __syncthreads();
  if (wave >= kWaves) return;

  // ---- 2. expand: out^T[d][b], d = d0 + 16 wave + 4 (lane / 16) + r, b = b0 + 16 bb + lane % 16
  constexpr int kBB = kRows / 16;
  const int bl = lane & 15, kg = lane >> 4;
  floatx4 acc[kBB];
#pragma unroll
  for (int bb = 0; bb < kBB; ++bb) acc[bb] = floatx4{};
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const half8 a = __builtin_bit_cast(half8, bf16x8_to_f16x8(wr[ks]));
#pragma unroll
    for (int bb = 0; bb < kBB; ++bb) {
      const int bi = 16 * bb + bl;
      const half8 bv = *reinterpret_cast<const half8*>(olds + bi * (kDc * 2) + 16 * ((4 * ks + kg) ^ bl));
      acc[bb] = mfma16x16x32(a, bv, acc[bb]);
    }
  }
  const int d = d0 + 16 * wave + 4 * kg;
#pragma unroll
  for (int bb = 0; bb < kBB; ++bb) {
    const int b = b0 + 16 * bb + bl;
    if (16 * bb + bl < kCoB && b < B) {
      u32x2 v;
      v[0] = (uint32_t)f32_to_bf16_rne(acc[bb][0]) | ((uint32_t)f32_to_bf16_rne(acc[bb][1]) << 16);
      v[1] = (uint32_t)f32_to_bf16_rne(acc[bb][2]) | ((uint32_t)f32_to_bf16_rne(acc[bb][3]) << 16);
      *reinterpret_cast<u32x2*>(out + ((int64_t)b * H + h) * kDn + d) = v;
      if (out_f32 != nullptr) *reinterpret_cast<floatx4*>(out_f32 + ((int64_t)b * H + h) * kDn + d) = acc[bb];
    }
  }
}

__global__ __launch_bounds__(256) void wo_kernel(const float* __restrict__ x, const uint16_t* __restrict__ w_o,
                                                 int K, int N, uint16_t* __restrict__ y, int B) {
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= N) return;
  const uint16_t* wr = w_o + (int64_t)n * K;
  for (int b = 0; b < B; ++b) {
    const float* xr = x + (int64_t)b * K;
    float acc = 0.f;
    for (int k = 8 * lane; k < K; k += 512) {
      const u32x4 wv = ld16(wr + k);
      const floatx4 x0 = *reinterpret_cast<const floatx4*>(xr + k);
      const floatx4 x1 = *reinterpret_cast<const floatx4*>(xr + k + 4);
      const float xs[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(__uint_as_float(wv[e] << 16), xs[2 * e], acc);              // element 2e (low half)
        acc = fmaf(__uint_as_float(wv[e] & 0xffff0000u), xs[2 * e + 1], acc);  // element 2e+1
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) y[(int64_t)b * N + n] = f32_to_bf16_rne(acc);
  }
}

}  // namespace

hipError_t launch_combine(int num_heads, const uint16_t* o_part, const float* lse_part, const int32_t* split_offsets,
                          float* o_lat, float* lse, int batch, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(batch * num_heads), dim3(128), 0, stream, o_part, lse_part, split_offsets,
                     o_lat, lse, num_heads);
  return hipGetLastError();
}

hipError_t launch_out_proj(int num_heads, const float* o_lat, const uint16_t* w_uv, uint16_t* out, float* out_f32,
                           int batch, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(out_proj_kernel, dim3(num_heads * 4), dim3(256), 0, stream, o_lat, w_uv, out, out_f32, num_heads,
                     batch);
  return hipGetLastError();
}

hipError_t launch_combine_out_proj(int num_heads, const uint16_t* o_part, const float* lse_part,
                                  const int32_t* split_offsets, const uint16_t* w_uv, uint16_t* out, float* out_f32,
                                  float* o_lat, float* lse, int batch, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  if (num_heads * ((batch + 31) / 32) >= 128)
    hipLaunchKernelGGL((combine_out_proj_kernel<32, 4, 1>), dim3(num_heads * ((batch + 31) / 32)), dim3(kCoThreads), 0,
                       stream, o_part, lse_part, split_offsets, w_uv, out, out_f32, o_lat, lse, num_heads, batch);
  else
    hipLaunchKernelGGL((combine_out_proj_kernel<8, 8, 4>), dim3(num_heads * ((batch + 7) / 8) * 4), dim3(kCoThreads), 0,
                       stream, o_part, lse_part, split_offsets, w_uv, out, out_f32, o_lat, lse, num_heads, batch);
  return hipGetLastError();
}

hipError_t launch_wo_proj(int in_features, const float* x, const uint16_t* w_o, int hidden, uint16_t* y, int batch,
                          hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(wo_kernel, dim3((hidden + 3) / 4), dim3(256), 0, stream, x, w_o, in_features, hidden, y, batch);
  return hipGetLastError();
}

}  // namespace mla
