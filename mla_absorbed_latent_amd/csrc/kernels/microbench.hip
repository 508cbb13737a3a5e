// microbench.hip -- what this card achieves on plain work, measured in the same
// run as the decode (achievable-peak context for the vendor figures), and its
// shader clock at a given moment.  Not part of the method: bench-only entry
// points declared in include/mla_bench.h.
//   * stream_read: every byte of a buffer read once with 16-byte loads (HBM
//     read bandwidth; one sum per work-group is written so nothing is elided);
//   * mfma_loop: independent chains of v_mfma_f32_32x32x16_{f16,bf16} on
//     register operands (matrix-core throughput with no memory traffic);
//   * cu_read: one 512-thread work-group per CU reads its own 64 KB slice over
//     and over (L2-resident when the slices fit), with plain 16-byte loads or
//     with direct-to-LDS loads, timing itself with the shader-clock counter:
//     the bytes a CU takes in per cycle from L2 on either path;
//   * clock_probe: one wave reads the shader-clock counter (s_memtime) and the
//     constant 100 MHz counter (s_memrealtime) around a fixed spin, giving the
//     shader clock over that interval.
#include "common.h"
#include "../../../include/mla_bench.h"

namespace mla {
namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                          uint32_t* __restrict__ out) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // four loads in flight per thread
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= (a[0] ^ a[1] ^ a[2] ^ a[3]) + (b[0] ^ b[1] ^ b[2] ^ b[3]) + (c[0] ^ c[1] ^ c[2] ^ c[3]) +
           (d[0] ^ d[1] ^ d[2] ^ d[3]);
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// Eight independent accumulator chains per wave; each MFMA depends on the one
// eight steps earlier, far more than the instruction's latency.
template <bool kBf16>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  half8 a, b;
  bf16x8 ab, bb;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (_Float16)(0.001f * (lane + j));
    b[j] = (_Float16)(0.002f * (lane - j));
    ab[j] = (__bf16)(0.001f * (lane + j));
    bb[j] = (__bf16)(0.002f * (lane - j));
  }
  floatx16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = floatx16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if constexpr (kBf16) acc[c] = mfma32x32x16_bf16(ab, bb, acc[c]);
      else acc[c] = mfma32x32x16(a, b, acc[c]);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Work-group b reads slice b (4,096 chunks of 16 B) iters times.  Plain: each
// thread keeps eight 16-byte loads in flight (its chunks t + 512 k, rotated by
// 64 per pass so that no load is hoisted out of the loop) and folds them into a
// sum.  Direct-to-LDS: wave w copies 1 KB segments w + 8 k of the slice into
// the work-group's 64 KB of LDS, waiting each second pass until one pass's
// loads are left in flight.  cycles[b] = shader cycles of the loop.
__global__ __launch_bounds__(512, 1) void cu_read_kernel(const u32x4* __restrict__ buf, int iters, int dma,
                                                         uint32_t* __restrict__ out, uint64_t* __restrict__ cycles) {
  __shared__ __attribute__((aligned(1024))) char lds[65536];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const u32x4* p = buf + (int64_t)blockIdx.x * 4096;
  u32x4 acc = {0u, 0u, 0u, 0u};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  if (dma) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int seg = wave + 8 * k;
        __builtin_amdgcn_global_load_lds(p + 64 * seg + lane, (__attribute__((address_space(3))) void*)(lds + 1024 * seg),
                                         16, 0, 0);
      }
      if (it & 1) __builtin_amdgcn_s_waitcnt((8 & 15) | (7 << 4) | (15 << 8));   // vmcnt(8)
    }
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));                              // vmcnt(0)
  } else {
    for (int it = 0; it < iters; ++it) {
      u32x4 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(p + ((512 * k + (int)threadIdx.x + 64 * it) & 4095));
#pragma unroll
      for (int k = 0; k < 8; ++k) acc += v[k];
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  __syncthreads();
  acc[0] += *reinterpret_cast<const uint32_t*>(lds + 4 * threadIdx.x);
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off, 64);
  if (lane == 0) out[(int64_t)blockIdx.x * 8 + wave] = x;
  if (threadIdx.x == 0) cycles[blockIdx.x] = t1 - t0;
}

__global__ __launch_bounds__(64) void clock_probe_kernel(int spins, uint64_t* __restrict__ out) {
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  uint32_t x = threadIdx.x;
  for (int i = 0; i < spins; ++i) x = x * 1664525u + 1013904223u;
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
    out[2] = x;
  }
}

hipError_t check_gfx950() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return e;
  return __builtin_strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? hipSuccess : hipErrorInvalidDeviceFunction;
}

}  // namespace
}  // namespace mla

extern "C" {

int32_t mla_bench_stream_read(const void* buf, int64_t bytes, uint32_t* out, int32_t blocks, hipStream_t stream) {
  if (!buf || !out || bytes < 16 || (bytes & 15) || blocks <= 0 || ((uintptr_t)buf & 15)) return (int32_t)hipErrorInvalidValue;
  hipError_t e = mla::check_gfx950();
  if (e != hipSuccess) return (int32_t)e;
  hipLaunchKernelGGL(mla::stream_read_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const mla::u32x4*>(buf), bytes / 16, out);
  return (int32_t)hipGetLastError();
}

int32_t mla_bench_mfma_loop(int32_t bf16, int32_t iters, int32_t blocks, float* out, hipStream_t stream) {
  if (!out || iters <= 0 || blocks <= 0) return (int32_t)hipErrorInvalidValue;
  hipError_t e = mla::check_gfx950();
  if (e != hipSuccess) return (int32_t)e;
  if (bf16) hipLaunchKernelGGL(mla::mfma_loop_kernel<true>, dim3(blocks), dim3(256), 0, stream, iters, out);
  else hipLaunchKernelGGL(mla::mfma_loop_kernel<false>, dim3(blocks), dim3(256), 0, stream, iters, out);
  return (int32_t)hipGetLastError();
}

int32_t mla_bench_cu_read(const void* buf, int32_t blocks, int32_t iters, int32_t dma, uint32_t* out,
                          uint64_t* cycles, hipStream_t stream) {
  if (!buf || !out || !cycles || blocks <= 0 || iters <= 0 || ((uintptr_t)buf & 15)) return (int32_t)hipErrorInvalidValue;
  hipError_t e = mla::check_gfx950();
  if (e != hipSuccess) return (int32_t)e;
  hipLaunchKernelGGL(mla::cu_read_kernel, dim3(blocks), dim3(512), 0, stream, static_cast<const mla::u32x4*>(buf),
                     iters, dma ? 1 : 0, out, cycles);
  return (int32_t)hipGetLastError();
}

int32_t mla_bench_clock_probe(int32_t spins, uint64_t* out, hipStream_t stream) {
  if (!out || spins <= 0) return (int32_t)hipErrorInvalidValue;
  hipError_t e = mla::check_gfx950();
  if (e != hipSuccess) return (int32_t)e;
  hipLaunchKernelGGL(mla::clock_probe_kernel, dim3(1), dim3(64), 0, stream, spins, out);
  return (int32_t)hipGetLastError();
}

}  // extern "C"
