// absorb.hip -- fold W_UK into the query ("DeepSeek MLA 吸收式缓存：真实权重执行与
// FlashMLA 架构边界" §2.2; "手搓 MLA:从 MHA 到 weight absorption" §四, einsum
// "thd,hdc->thc"):
//     q_abs[b,h,c]       = sum_d q_nope[b,h,d] * W_UK[h,d,c]     c < 512
//     q_abs[b,h,512 + r] = q_pe[b,h,r]
//
// Per head this is a [B x 128] x [128 x 512] product.  It runs transposed on the
// bf16 matrix cores (bf16 x bf16 products are exact in the fp32 accumulator):
//     q_abs^T[c][b] = W_UK[h]^T[c][d] . q_nope^T[d][b]      (mfma 32x32x16 bf16)
// A work-group owns one head and 128 latent columns.  W_UK[h][:, c0:c0+128] is
// staged row-major in LDS and read transposed (ds_read_b64_tr_b16), so every
// lane gets 8 consecutive d for its column c; q_nope rows come straight from
// HBM as 16-byte loads.  The result is rounded to fp16 (round to nearest even)
// and stored 4 consecutive columns at a time.
#include "common.h"
#include "kernels.h"

namespace mla {
namespace {

constexpr int kSlab = 128;                       // latent columns per work-group
constexpr int kWRow = kSlab * 2;                 // 256 B per LDS row (one d)

__global__ __launch_bounds__(256) void absorb_q_kernel(const uint16_t* __restrict__ q_nope,
                                                       const uint16_t* __restrict__ q_pe,
                                                       const uint16_t* __restrict__ w_uk,
                                                       uint16_t* __restrict__ q_abs, int H, int B,
                                                       uint8_t* __restrict__ pool, int64_t num_pages,
                                                       const uint16_t* __restrict__ c_kv,
                                                       const uint16_t* __restrict__ k_pe,
                                                       const int64_t* __restrict__ slots, int n_new) {
  // Work-groups past the absorb grid append the step's new tokens to a bf16
  // cache (16-byte chunk `chunk` of token `tok`'s 1,152-byte row), so that a
  // decode step's append and absorb take one launch.  Out-of-range slots are
  // skipped, as in mla_cache_append.
  const int n_absorb = H * (kDc / kSlab);
  if ((int)blockIdx.x >= n_absorb) {
    const int64_t gid = (int64_t)(blockIdx.x - n_absorb) * 256 + threadIdx.x;
    const int64_t tok = gid / 72;
    const int chunk = (int)(gid % 72);
    if (tok >= n_new) return;
    const uint16_t* src = chunk < 64 ? c_kv + tok * kDc + chunk * 8 : k_pe + tok * kDr + (chunk - 64) * 8;
    const u32x4 v = ld16(src);
    const int64_t slot = slots[tok];
    if (slot < 0 || slot >= num_pages * kBlock) return;
    st16(pool + (slot / kBlock) * (kBlock * kRowBytesBf16) + (slot % kBlock) * kRowBytesBf16 + chunk * 16, v);
    return;
  }
  __shared__ __attribute__((aligned(16))) char lds[kDn * kWRow];     // 32 KB
  // Output tile of 32 sequences x 128 columns (fp16, rows of 256 B, 16-byte chunk c
  // at c ^ (row & 15)): written in the accumulator layout, read back as whole
  // 256-byte row pieces so that the q_abs stores are contiguous.
  __shared__ __attribute__((aligned(16))) char otile[32 * kWRow];    // 8 KB
  const int h = blockIdx.x / (kDc / kSlab);
  const int c0 = (blockIdx.x % (kDc / kSlab)) * kSlab;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // Stage W_UK[h][0:128][c0:c0+128] (128 rows x 16 chunks of 16 B): all eight
  // loads of a thread, and the q_nope rows of the first 32 sequences, are issued
  // before any LDS write, so they overlap.
  const uint16_t* wsrc = w_uk + (int64_t)h * kDn * kDc + c0;
  u32x4 wv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = threadIdx.x + 256 * i, d = idx >> 4, ch = idx & 15;
    wv[i] = ld16(wsrc + (int64_t)d * kDc + 8 * ch);
  }
  const int g = lane >> 5, grp = lane >> 4, gi = lane & 15;
  // q_nope[b][h][16 ks + 8 g .. +7] for b = b0 + lane % 32 (a sequence past B
  // reads row 0 instead; its column is never stored).
  auto load_q = [&](int b0, u32x4 (&qa)[kDn / 16]) {
    const int b = b0 + (lane & 31);
    const uint16_t* qrow = q_nope + ((int64_t)(b < B ? b : 0) * H + h) * kDn + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kDn / 16; ++ks) qa[ks] = ld16(qrow + 16 * ks);
  };
  u32x4 qa[kDn / 16];
  load_q(0, qa);
  // q_pe passthrough (bf16 -> fp16 is exact in range): the four slab work-groups of
  // a head share it, sequence b going to slab b % 4; its loads join the ones above.
  {
    const int slab = c0 / kSlab, nb = (B - slab + 3) / 4;
    for (int i = threadIdx.x; i < nb * 8; i += 256) {
      const int b = slab + 4 * (i >> 3), ch = i & 7;
      const u32x4 v = ld16(q_pe + ((int64_t)b * H + h) * kDr + 8 * ch);
      st16(q_abs + ((int64_t)b * H + h) * kDk + kDc + 8 * ch, bf16x8_to_f16x8(v));
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = threadIdx.x + 256 * i, d = idx >> 4, ch = idx & 15;
    *reinterpret_cast<u32x4*>(lds + d * kWRow + 16 * (ch ^ (d & 7))) = wv[i];
  }
  __syncthreads();

  // Transposed read: group lane gi addresses row (d) d0 + (gi >> 2), columns
  // 16 (grp & 1) + 4 (gi & 3) of this wave's 32-column block.
  const int cw = 32 * wave;                            // wave's columns within the slab
  const int colh = cw + 16 * (grp & 1) + 4 * (gi & 3);  // in halves
  for (int b0 = 0; b0 < B; b0 += 32) {
    floatx16 acc = floatx16{};
    u32x4 qn[kDn / 16];                                // the next 32 sequences, in flight meanwhile
    if (b0 + 32 < B) load_q(b0 + 32, qn);
#pragma unroll
    for (int ks = 0; ks < kDn / 16; ++ks) {
      const u32x4 qv = qa[ks];
      const int d = 16 * ks + 8 * g + (gi >> 2);
      const int ch = colh >> 3;
      const uint32_t off_lo = d * kWRow + 16 * (ch ^ (d & 7)) + 2 * (colh & 7);
      const int d4 = d + 4;
      const uint32_t off_hi = d4 * kWRow + 16 * (ch ^ (d4 & 7)) + 2 * (colh & 7);
      const half4 lo = lds_read_tr(lds, off_lo);
      const half4 hi = lds_read_tr(lds, off_hi);
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc = mfma32x32x16_bf16(a, __builtin_bit_cast(bf16x8, qv), acc);
    }
    // lane holds columns cw + 8 rr + 4 g + 0..3 of sequence b0 + lane % 32
    const int bl = lane & 31;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      u32x2 v;
      v[0] = (uint32_t)f32_to_f16_bits(acc[4 * rr]) | ((uint32_t)f32_to_f16_bits(acc[4 * rr + 1]) << 16);
      v[1] = (uint32_t)f32_to_f16_bits(acc[4 * rr + 2]) | ((uint32_t)f32_to_f16_bits(acc[4 * rr + 3]) << 16);
      *reinterpret_cast<u32x2*>(otile + bl * kWRow + 16 * (((cw >> 3) + rr) ^ (bl & 15)) + 8 * g) = v;
    }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int row = 16 * pass + (threadIdx.x >> 4), chunk = threadIdx.x & 15;
      const u32x4 v = *reinterpret_cast<const u32x4*>(otile + row * kWRow + 16 * (chunk ^ (row & 15)));
      if (b0 + row < B) st16(q_abs + ((int64_t)(b0 + row) * H + h) * kDk + c0 + 8 * chunk, v);
    }
    __syncthreads();                                   // the tile is free for the next 32 sequences
    if (b0 + 32 < B) {
#pragma unroll
      for (int ks = 0; ks < kDn / 16; ++ks) qa[ks] = qn[ks];
    }
  }
}

}  // namespace

hipError_t launch_absorb_q(int num_heads, const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* w_uk,
                           uint16_t* q_abs, int batch, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(absorb_q_kernel, dim3(num_heads * (kDc / kSlab)), dim3(256), 0, stream, q_nope, q_pe, w_uk,
                     q_abs, num_heads, batch, nullptr, (int64_t)0, nullptr, nullptr, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_append_absorb(int cache_dtype, void* pool, int64_t num_pages, const uint16_t* c_kv,
                                const uint16_t* k_pe, const int64_t* slots, int n_new, int num_heads,
                                const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* w_uk, uint16_t* q_abs,
                                int batch, hipStream_t stream) {
  if (cache_dtype != 0 || batch <= 0 || n_new <= 0) {
    hipError_t e = launch_append(cache_dtype, pool, num_pages, c_kv, k_pe, slots, n_new, stream);
    if (e != hipSuccess) return e;
    return launch_absorb_q(num_heads, q_nope, q_pe, w_uk, q_abs, batch, stream);
  }
  const int64_t append_blocks = ((int64_t)n_new * 72 + 255) / 256;
  hipLaunchKernelGGL(absorb_q_kernel, dim3((unsigned)(num_heads * (kDc / kSlab) + append_blocks)), dim3(256), 0,
                     stream, q_nope, q_pe, w_uk, q_abs, num_heads, batch, static_cast<uint8_t*>(pool), num_pages,
                     c_kv, k_pe, slots, n_new);
  return hipGetLastError();
}

}  // namespace mla
