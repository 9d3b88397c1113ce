/*
 * Practical ceilings of MI355X (gfx950) for the decode's rooflines: C
 * interface of the calibration kernels that bench.py's --ceiling modes time.
 * They are not part of the decode path. The decode's arithmetic is bf16
 * MFMA and its data movement is HBM -> LDS page copies (FlashAttention (KO),
 * "GPU 메모리 계층 구조": the gap between on-chip memory and HBM sets the
 * speed of attention); these kernels measure what the chip delivers for
 * each with the same instructions, next to the nominal peaks (dense bf16
 * MFMA 2.5 PFLOP/s, HBM 8 TB/s).
 *
 * Pointers are device pointers; work is enqueued on `stream`; nothing is
 * allocated or synchronised. Return 0, or a negative MLA_CEIL_ERR_* code
 * (argument checks run before anything is enqueued).
 */
#ifndef MLA_CEILING_H_
#define MLA_CEILING_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MLA_CEIL_ERR_ARG = -2, MLA_CEIL_ERR_HIP = -5 };

/* bf16 MFMA throughput with register operands. kind 0: 16x16x32
 * (16384 flop per instruction; accumulators 4 or 8); kind 1: 32x32x16
 * (32768 flop; accumulators 2 or 4). Each wave issues iters * accumulators
 * independent MFMAs; grid * waves_per_simd workgroups of 4 waves (one per
 * SIMD of a CU when grid is the CU count; waves_per_simd 1 or 2).
 * sink: fp32 [grid * waves_per_simd * 256], written once per thread. */
int mla_ceiling_mfma(int32_t kind, int32_t accumulators, int32_t waves_per_simd, int32_t iters,
                     int32_t grid, float* sink, hipStream_t stream);

/* Read `bytes` (a multiple of 16, src 16-byte aligned) once with
 * non-temporal 16-byte loads, grid workgroups of 256 threads striding over
 * the buffer. sink: uint32 [grid * 256]. */
int mla_ceiling_stream_read(const void* src, size_t bytes, int32_t grid, uint32_t* sink,
                            hipStream_t stream);

/* Copy every whole 72 KiB block of src (bytes / 73728 blocks) into LDS with
 * global_load_lds_dwordx4, the way the decode copies a latent page: grid
 * workgroups of `waves` waves (4 or 8) take blocks grid apart, double
 * buffered, one wait and one barrier per block, no other work.
 * sink: uint32 [grid]. */
int mla_ceiling_lds_fill(const void* src, size_t bytes, int32_t waves, int32_t grid,
                         uint32_t* sink, hipStream_t stream);

/* LDS operand reads, alone and as MFMA operands. Every wave reads 1 KiB of
 * LDS per step, iters * 16 steps: mode 0 one ds_read_b128 per lane; mode 1
 * the same read as the A operand of a 32x32x16 bf16 MFMA (32768 flop);
 * mode 2 two ds_read_b64_tr_b16 per lane feeding the MFMA; mode 3 those two
 * reads alone; modes 4 and 5 are modes 1 and 2 with each read issued
 * eight steps before its MFMA. grid workgroups of `waves` waves (4 or 8), each with 64 KiB
 * of LDS. sink: fp32 [grid * 64 * waves]. */
int mla_ceiling_lds_operand(int32_t mode, int32_t waves, int32_t iters, int32_t grid, float* sink,
                            hipStream_t stream);

/* Write block_bytes (a multiple of 16) at dst + w * stride_bytes for each
 * workgroup w < grid (256 threads, 16-byte stores, lanes consecutive): the
 * HBM write rate for one block per workgroup, and how it depends on the
 * blocks' spacing. dst must hold (grid - 1) * stride_bytes + block_bytes. */
int mla_ceiling_block_write(void* dst, size_t block_bytes, size_t stride_bytes, int32_t grid,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif  // MLA_CEILING_H_
