// combine_out.hip -- log-sum-exp merge of split-KV partials, and the output
// projections.
//
// Merge (one work-group per (sequence, head); exact for any split of the tokens):
//     lse = ln sum_j e^{lse_j},  o_lat = sum_j e^{lse_j - lse} o_j
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
// One wave per (head, 32 rows of d); the fp32 sums go to `out` as bf16 and,
// when a layer output is wanted, to an fp32 workspace for the W_O product.
//
// W_O product (optional): y[b,n] = sum_k W_O[n,k] x[b,k], x = concat_h out[b,h,:]
// in fp32; one wave per output feature, fp32 FMAs, a wave reduction.
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      const int32_t* __restrict__ offsets, float* __restrict__ o_lat,
                                                      float* __restrict__ lse_out, int H) {
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int r0 = offsets[b], r1 = offsets[b + 1];
  float m = -INFINITY;
  for (int j = r0; j < r1; ++j) m = fmaxf(m, lse_part[(int64_t)j * H + h]);
  floatx4 acc = floatx4{};
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int j = r0; j < r1; ++j) {
      const float l = lse_part[(int64_t)j * H + h];
      if (l == -INFINITY) continue;
      const float w = expf(l - m);
      wsum += w;
      acc += w * *reinterpret_cast<const floatx4*>(o_part + ((int64_t)j * H + h) * kDc + 4 * threadIdx.x);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  *reinterpret_cast<floatx4*>(o_lat + ((int64_t)b * H + h) * kDc + 4 * threadIdx.x) = acc * inv;
  if (lse_out != nullptr && threadIdx.x == 0) lse_out[(int64_t)b * H + h] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
}

__global__ __launch_bounds__(64) void out_proj_kernel(const float* __restrict__ o_lat, const uint16_t* __restrict__ w_uv,
                                                      uint16_t* __restrict__ out, float* __restrict__ out_f32, int H,
                                                      int B) {
  const int h = blockIdx.x >> 2;
  const int d0 = (blockIdx.x & 3) * 32;
  const int lane = threadIdx.x;
  const int g = lane >> 5;
  const uint16_t* wrow = w_uv + ((int64_t)h * kDn + d0 + (lane & 31)) * kDc + 8 * g;
  for (int b0 = 0; b0 < B; b0 += 32) {
    const int b = b0 + (lane & 31);
    const bool bok = b < B;
    const float* orow = o_lat + ((int64_t)(bok ? b : 0) * H + h) * kDc + 8 * g;
    floatx16 acc = floatx16{};
#pragma unroll 4
    for (int ks = 0; ks < kDc / 16; ++ks) {
      const half8 a = __builtin_bit_cast(half8, bf16x8_to_f16x8(ld16(wrow + 16 * ks)));
      half8 bv;
      if (bok) {
        const floatx4 x0 = *reinterpret_cast<const floatx4*>(orow + 16 * ks);
        const floatx4 x1 = *reinterpret_cast<const floatx4*>(orow + 16 * ks + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bv[e] = (_Float16)x0[e];
          bv[4 + e] = (_Float16)x1[e];
        }
      } else {
        bv = half8{};
      }
      acc = mfma32x32x16(a, bv, acc);
    }
    if (bok) {
      // lane holds out^T[d0 + 8 (r/4) + 4 g + r%4][b]
      uint16_t* dst = out + ((int64_t)b * H + h) * kDn + d0 + 4 * g;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        u32x2 v;
        v[0] = (uint32_t)f32_to_bf16_rne(acc[4 * rr]) | ((uint32_t)f32_to_bf16_rne(acc[4 * rr + 1]) << 16);
        v[1] = (uint32_t)f32_to_bf16_rne(acc[4 * rr + 2]) | ((uint32_t)f32_to_bf16_rne(acc[4 * rr + 3]) << 16);
        *reinterpret_cast<u32x2*>(dst + 8 * rr) = v;
        if (out_f32 != nullptr) {
          float* fd = out_f32 + ((int64_t)b * H + h) * kDn + d0 + 4 * g + 8 * rr;
          *reinterpret_cast<floatx4*>(fd) = floatx4{acc[4 * rr], acc[4 * rr + 1], acc[4 * rr + 2], acc[4 * rr + 3]};
        }
      }
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

hipError_t launch_combine(int num_heads, const float* o_part, const float* lse_part, const int32_t* split_offsets,
                          float* o_lat, float* lse, int batch, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(batch * num_heads), dim3(128), 0, stream, o_part, lse_part, split_offsets,
                     o_lat, lse, num_heads);
  return hipGetLastError();
}

hipError_t launch_out_proj(int num_heads, const float* o_lat, const uint16_t* w_uv, uint16_t* out, float* out_f32,
                           int batch, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(out_proj_kernel, dim3(num_heads * 4), dim3(64), 0, stream, o_lat, w_uv, out, out_f32, num_heads,
                     batch);
  return hipGetLastError();
}

hipError_t launch_wo_proj(int in_features, const float* x, const uint16_t* w_o, int hidden, uint16_t* y, int batch,
                          hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(wo_kernel, dim3((hidden + 3) / 4), dim3(256), 0, stream, x, w_o, in_features, hidden, y, batch);
  return hipGetLastError();
}

}  // namespace mla
