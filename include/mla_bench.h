/*
 * mla_bench.h -- measurement helpers of the absorbed-latent MLA library
 * (gfx950): what the card achieves on plain work in the same run as the
 * decode, and its shader clock at a given moment.  They are context for the
 * decode's roofline figures and take no part in the method.  Each call is
 * asynchronous on `stream`, returns a hipError_t value (0 on success), checks
 * that the current device is gfx950, and reads or writes only the buffers
 * given; the caller owns every buffer.
 */
#ifndef MLA_BENCH_H
#define MLA_BENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

/* Reads every byte of buf once with 16-byte non-temporal loads (HBM read
 * bandwidth) using `blocks` work-groups of 256 threads, and writes one 32-bit
 * XOR per work-group to out[0 .. blocks-1].  buf 16-byte aligned, bytes a
 * positive multiple of 16.                                                   */
int32_t mla_bench_stream_read(const void* buf, int64_t bytes, uint32_t* out, int32_t blocks, hipStream_t stream);

/* Matrix-core throughput: `blocks` work-groups of four waves, each wave issuing
 * iters x 8 independent v_mfma_f32_32x32x16_f16 (bf16 != 0: _bf16) on register
 * operands, i.e. 2 * 32 * 32 * 16 * 8 * iters FLOP per wave; writes one float
 * per thread to out[0 .. 256 * blocks - 1].                                  */
int32_t mla_bench_mfma_loop(int32_t bf16, int32_t iters, int32_t blocks, float* out, hipStream_t stream);

/* Per-CU read rate from L2: `blocks` work-groups of 512 threads (size it to one
 * per CU), work-group b reading bytes 65536 b .. 65536 b + 65535 of buf
 * `iters` times, with 16-byte loads into registers (dma == 0, eight in
 * flight per thread) or with direct-to-LDS 16-byte loads (dma != 0).  With
 * blocks x 64 KB within the L2s the slices stay resident after the first
 * pass.  Writes cycles[b] = shader-clock cycles of work-group b's loop (so
 * iters x 65536 / cycles[b] is bytes per cycle for that CU) and one 32-bit
 * value per wave to out[0 .. 8 * blocks - 1] (kept so nothing is elided).
 * buf: 65536 * blocks bytes, 16-byte aligned.                               */
int32_t mla_bench_cu_read(const void* buf, int32_t blocks, int32_t iters, int32_t dma, uint32_t* out,
                          uint64_t* cycles, hipStream_t stream);

/* Shader clock: one wave spins `spins` dependent integer steps between two
 * reads of the shader-clock counter and of the constant 100 MHz counter;
 * writes out[0] = shader cycles, out[1] = 100 MHz ticks, out[2] = a value of
 * the spin (kept so it is not elided).  Clock = out[0] / out[1] * 100 MHz.  */
int32_t mla_bench_clock_probe(int32_t spins, uint64_t* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MLA_BENCH_H */
