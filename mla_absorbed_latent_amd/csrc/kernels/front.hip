// front.hip -- the layer front that produces the hot path's inputs from a
// layer's hidden states (V2-Lite shapes):
//   * one query projection and one joint down projection whose output puts the
//     512-wide latent first, then the 64-wide RoPE key
//     ("DeepSeek-V2-Lite MLA 吸收式 KV 缓存优化 — 完整实验报告" §1.1;
//      "DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界" §3.3);
//   * the latent is RMS-normalised before it is cached, the RoPE key and the
//     query's RoPE part are rotated by position
//     ("手搓 MLA:从 MHA 到 weight absorption,看懂 DeepSeek 的 KV 压缩" §三).
// Readings where the pages are silent: RMSNorm with unit gain; RoPE on
// interleaved pairs (x[2i], x[2i+1]) rotated by pos * base^(-2i/64); every
// output rounded once to bf16.
//
// launch_out_residual closes a layer: x += W_O . attention output, with the
// same rowdot kernel for W_O and an elementwise residual kernel.
//
// The projections y[t][n] = sum_k W[n][k] x[t][k] (bf16 in, fp32 sums) take one
// of two kernels: rowdot for a few tokens (a decode step: weight-read-bound, on
// the vector ALUs with one wave per output feature) and gemm_nt for chunks of
// 64 tokens or more (a prompt: compute-bound, on the matrix cores); then
// front_finish applies the norm, the rotation and the bf16 rounding (the norm
// and the angles in double precision).
#include <atomic>
#include <mutex>

#include "append_row.h"
#include "common.h"
#include "kernels.h"

namespace mla {

// Device scratch of launch_layer_front_noalloc: the fp32 projections that
// launch_layer_front otherwise keeps in the caller's workspace.  Every GPU the
// library runs on holds its own copy until the process ends; every call on a
// GPU shares it.  The projections write every element they later read, so it
// needs no clearing between calls.
__device__ __attribute__((aligned(256))) static float scratch[kFrontScratchBytes / sizeof(float)];

namespace {

constexpr int kTokChunk = 16;      // tokens accumulated together per pass over a weight row

__device__ __forceinline__ float dot8_bf16(u32x4 a, u32x4 b) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s = fmaf(__uint_as_float(a[e] << 16), __uint_as_float(b[e] << 16), s);
    s = fmaf(__uint_as_float(a[e] & 0xffff0000u), __uint_as_float(b[e] & 0xffff0000u), s);
  }
  return s;
}

// One wave per output feature n (four per work-group); lane l reads the 16-byte
// chunks 8 l + 512 j of the weight row and of each token's row.
__global__ __launch_bounds__(256) void rowdot_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                     int K, int N, int T, float* __restrict__ y) {
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= N) return;
  const uint16_t* wr = w + (int64_t)n * K;
  for (int t0 = 0; t0 < T; t0 += kTokChunk) {
    float acc[kTokChunk];
#pragma unroll
    for (int i = 0; i < kTokChunk; ++i) acc[i] = 0.f;
    for (int k = 8 * lane; k < K; k += 512) {
      const u32x4 wv = ld16(wr + k);
#pragma unroll
      for (int i = 0; i < kTokChunk; ++i) {
        const int t = t0 + i < T ? t0 + i : T - 1;     // rows past T are read again and dropped
        acc[i] += dot8_bf16(wv, ld16(x + (int64_t)t * K + k));
      }
    }
#pragma unroll
    for (int i = 0; i < kTokChunk; ++i) {
      float v = acc[i];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
      if (lane == 0 && t0 + i < T) y[(int64_t)(t0 + i) * N + n] = v;
    }
  }
}

// y[t][n] = sum_k x[t][k] w[n][k] on the matrix cores, for chunks of many
// tokens: a work-group computes 128 tokens x 128 features from 64-channel
// chunks of both operands loaded straight into LDS (double-buffered, 16-byte
// chunk c of row r at c ^ (r & 7)); wave (wm, wn) holds 64 x 64 of the result
// as 4 x 4 tiles of v_mfma_f32_16x16x32_bf16.  K a multiple of 64; rows past T
// or N are not stored.
constexpr int kGT = 128;
constexpr int kGChunk = 64;
constexpr int kGRow = kGChunk * 2;               // 128 B
constexpr int kGBuf = 2 * kGT * kGRow;           // 32 KB

__global__ __launch_bounds__(256) void gemm_nt_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                      int K, int N, int T, float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kGBuf];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  const int t0 = blockIdx.y * kGT, n0 = blockIdx.x * kGT;
  // rows 0..127 x, 128..255 w, 8 chunks of 16 B per row, straight into LDS
  // (global_load_lds_dwordx4 fills a 1 KB segment, lane i bytes 16 i ..): 32
  // segments, wave w issues w + 4 i, each lane the chunk that belongs at its
  // slot.  Rows past T or N load row T - 1 or N - 1; their results are dropped.
  auto issue = [&](int kc, int buf) {
    char* base = lds + buf * kGBuf;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int seg = wave + 4 * i, P = 64 * seg + lane, row = P >> 3, ch = (P & 7) ^ (row & 7);
      const int k = kc * kGChunk + 8 * ch;
      const uint16_t* src;
      if (row < kGT) {
        const int t = t0 + row;
        src = x + (int64_t)(t < T ? t : T - 1) * K + k;
      } else {
        const int n = n0 + row - kGT;
        src = w + (int64_t)(n < N ? n : N - 1) * K + k;
      }
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(base + 1024 * seg), 16, 0, 0);
    }
  };
  floatx4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int n_chunks = K / kGChunk;
  issue(0, 0);
  for (int kc = 0; kc < n_chunks; ++kc) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();                       // chunk kc in LDS; chunk kc - 1 read by every wave
    if (kc + 1 < n_chunks) issue(kc + 1, (kc + 1) & 1);
    const char* buf = lds + (kc & 1) * kGBuf;
#pragma unroll
    for (int ks = 0; ks < kGChunk / 32; ++ks) {
      u32x4 xf[4], wf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int xr = 64 * wm + 16 * i + li, wr = kGT + 64 * wn + 16 * i + li;
        xf[i] = *reinterpret_cast<const u32x4*>(buf + xr * kGRow + 16 * ((4 * ks + g) ^ (xr & 7)));
        wf[i] = *reinterpret_cast<const u32x4*>(buf + wr * kGRow + 16 * ((4 * ks + g) ^ (wr & 7)));
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xf[a]),
                                                              __builtin_bit_cast(bf16x8, wf[b]), acc[a][b], 0, 0, 0);
    }
  }
  // D[token 64 wm + 16 a + 4 g + r][feature 64 wn + 16 b + li]
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int n = n0 + 64 * wn + 16 * b + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 64 * wm + 16 * a + 4 * g + r;
        if (t < T && n < N) y[(int64_t)t * N + n] = acc[a][b][r];
      }
    }
}

// y = x . w^T through the matrix-core tiles for chunks of 64 tokens or more
// (K a multiple of 64), else through rowdot.
void project(const uint16_t* x, const uint16_t* w, int K, int N, int T, float* y, hipStream_t stream) {
  if (T >= 64 && K % kGChunk == 0)
    hipLaunchKernelGGL(gemm_nt_kernel, dim3((N + kGT - 1) / kGT, (T + kGT - 1) / kGT), dim3(256), 0, stream, x, w,
                       K, N, T, y);
  else
    hipLaunchKernelGGL(rowdot_kernel, dim3((N + 3) / 4), dim3(256), 0, stream, x, w, K, N, T, y);
}

__device__ __forceinline__ uint16_t bf16_of(double v) { return f32_to_bf16_rne((float)v); }

// One work-group (256 threads) per token t: the 32 rotation angles of its
// position are evaluated once (double precision) into LDS and shared by the
// RoPE key and the H query heads; wave 0 normalises the latent.  With a pool
// (formats 0-6), the group then writes the token's row into its cache slot in
// the cache's format (the append kernels' own row functions, from an LDS copy of
// the row); slots outside the pool are skipped, as by mla_cache_append.
__global__ __launch_bounds__(256) void front_finish_kernel(const float* __restrict__ kv, const float* __restrict__ q,
                                                           const int32_t* __restrict__ pos, int H, float eps,
                                                           float base, uint16_t* __restrict__ q_nope,
                                                           uint16_t* __restrict__ q_pe, uint16_t* __restrict__ c_kv,
                                                           uint16_t* __restrict__ k_pe, int cache_dtype,
                                                           uint8_t* __restrict__ pool, int64_t num_pages,
                                                           const int64_t* __restrict__ slots, int n_tokens) {
  __shared__ double cs[32][2];
  __shared__ __attribute__((aligned(16))) uint16_t crow[kDc];
  __shared__ __attribute__((aligned(16))) uint16_t krow[kDr];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < 32) {
    // pair i of a 64-wide rotary vector turns by pos * base^(-2i/64)
    const double ang = (double)pos[t] * pow((double)base, -2.0 * tid / 64.0);
    cs[tid][0] = cos(ang);
    cs[tid][1] = sin(ang);
  }
  const float* kv_row = kv + (int64_t)t * (kDc + kDr);
  if (tid < 64) {
    double v[8], ss = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = kv_row[8 * tid + i];
      ss += v[i] * v[i];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const double inv = 1.0 / sqrt(ss / kDc + (double)eps);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint16_t b = bf16_of(v[i] * inv);
      c_kv[(int64_t)t * kDc + 8 * tid + i] = b;
      crow[8 * tid + i] = b;
    }
  }
  const float* q_tok = q + (int64_t)t * H * (kDn + kDr);
  for (int idx = tid; idx < H * kDn; idx += 256) {
    const int h = idx >> 7, d = idx & (kDn - 1);
    q_nope[((int64_t)t * H + h) * kDn + d] = bf16_of(q_tok[h * (kDn + kDr) + d]);
  }
  __syncthreads();
  // rotations: index H * 32 + i is pair i of the RoPE key, h * 32 + i of head h
  for (int idx = tid; idx < (H + 1) * 32; idx += 256) {
    const int h = idx >> 5, i = idx & 31;
    const float* src = h < H ? q_tok + h * (kDn + kDr) + kDn : kv_row + kDc;
    uint16_t* dst = h < H ? q_pe + ((int64_t)t * H + h) * kDr : k_pe + (int64_t)t * kDr;
    const double c = cs[i][0], sn = cs[i][1];
    const double xe = src[2 * i], xo = src[2 * i + 1];
    const uint16_t re = bf16_of(xe * c - xo * sn), ro = bf16_of(xe * sn + xo * c);
    dst[2 * i] = re;
    dst[2 * i + 1] = ro;
    if (h == H) {
      krow[2 * i] = re;
      krow[2 * i + 1] = ro;
    }
  }
  if (pool == nullptr) return;             // uniform: no append requested
  __syncthreads();                         // the row is complete in LDS
  const int64_t slot = slots[t];
  if (!slot_ok(slot, num_pages)) return;   // uniform per group
  append_row_wg(cache_dtype, pool, slot, crow, krow, tid);
}

// x_out[t][n] = bf16(x_in[t][n] + y[t][n]) (fp32 sum, round to nearest even);
// x_out may be x_in.
__global__ __launch_bounds__(256) void residual_kernel(const uint16_t* x_in, const float* __restrict__ y,
                                                       uint16_t* x_out, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    x_out[i] = f32_to_bf16_rne(bf16_to_f32(x_in[i]) + y[i]);
}

}  // namespace

hipError_t launch_out_residual(int num_heads, const uint16_t* attn_out, const uint16_t* w_o, int hidden,
                               const uint16_t* x_in, uint16_t* x_out, float* workspace, int n_tokens,
                               hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  project(attn_out, w_o, num_heads * kDn, hidden, n_tokens, workspace, stream);
  const int64_t n = (int64_t)n_tokens * hidden;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(residual_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, stream, x_in,
                     workspace, x_out, n);
  return hipGetLastError();
}

hipError_t launch_layer_front(int num_heads, const uint16_t* x, int hidden, const uint16_t* w_q, const uint16_t* w_dkv,
                              const int32_t* positions, float rms_eps, float rope_base, float* workspace,
                              uint16_t* q_nope, uint16_t* q_pe, uint16_t* c_kv, uint16_t* k_pe, int n_tokens,
                              hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  const int n_kv = kDc + kDr, n_q = num_heads * (kDn + kDr);
  float* kv = workspace;
  float* q = workspace + (int64_t)n_tokens * n_kv;
  project(x, w_dkv, hidden, n_kv, n_tokens, kv, stream);
  project(x, w_q, hidden, n_q, n_tokens, q, stream);
  hipLaunchKernelGGL(front_finish_kernel, dim3(n_tokens), dim3(256), 0, stream, kv, q, positions,
                     num_heads, rms_eps, rope_base, q_nope, q_pe, c_kv, k_pe, 0, nullptr, (int64_t)0, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_layer_front_append(int num_heads, const uint16_t* x, int hidden, const uint16_t* w_q,
                                     const uint16_t* w_dkv, const int32_t* positions, float rms_eps, float rope_base,
                                     float* workspace, uint16_t* q_nope, uint16_t* q_pe, uint16_t* c_kv,
                                     uint16_t* k_pe, int cache_dtype, void* pool, int64_t num_pages,
                                     const int64_t* slots, int n_tokens, hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  const int n_kv = kDc + kDr, n_q = num_heads * (kDn + kDr);
  float* kv = workspace;
  float* q = workspace + (int64_t)n_tokens * n_kv;
  project(x, w_dkv, hidden, n_kv, n_tokens, kv, stream);
  project(x, w_q, hidden, n_q, n_tokens, q, stream);
  // The per-channel INT8 format appends after the front, as mla_cache_append
  // does: a call that closes a block and opens the next one on the same page
  // must close first, since the new open rows take the overflow rows that the
  // closing block's earlier rows still occupy.
  const bool fuse = cache_dtype != 7;
  hipLaunchKernelGGL(front_finish_kernel, dim3(n_tokens), dim3(256), 0, stream, kv, q, positions, num_heads, rms_eps,
                     rope_base, q_nope, q_pe, c_kv, k_pe, cache_dtype, fuse ? static_cast<uint8_t*>(pool) : nullptr,
                     num_pages, slots, n_tokens);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && !fuse) e = launch_append(cache_dtype, pool, num_pages, c_kv, k_pe, slots, n_tokens, stream);
  return e;
}

// Device address of `scratch` on the current device, looked up once per device
// (the name is a host-side stand-in; only this address is valid on the GPU).
static hipError_t front_scratch(float** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<float*> addr[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* q = nullptr;
      e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (q == nullptr) return hipErrorInvalidSymbol;
      p = static_cast<float*>(q);
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_layer_front_noalloc(int num_heads, const uint16_t* x, int hidden, const uint16_t* w_q,
                                      const uint16_t* w_dkv, const int32_t* positions, float rms_eps,
                                      float rope_base, uint16_t* q_nope, uint16_t* q_pe, uint16_t* c_kv,
                                      uint16_t* k_pe, int n_tokens, hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  if ((size_t)n_tokens * (size_t)(kDc + kDr + num_heads * (kDn + kDr)) * sizeof(float) > kFrontScratchBytes)
    return hipErrorInvalidValue;     // the host entry point rejects this first
  float* ws = nullptr;
  const hipError_t e = front_scratch(&ws);
  if (e != hipSuccess) return e;
  return launch_layer_front(num_heads, x, hidden, w_q, w_dkv, positions, rms_eps, rope_base, ws, q_nope, q_pe,
                            c_kv, k_pe, n_tokens, stream);
}

}  // namespace mla
