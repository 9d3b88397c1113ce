// Practical ceilings of the chip for the decode's two rooflines, measured
// with the same instructions the decode uses:
//   * mfma_loop_kernel: bf16 MFMA throughput with operands in registers
//     (16x16x32 or 32x32x16, several independent accumulators per wave),
//     the attainable compute rate next to the nominal dense peak;
//   * stream_read_kernel: HBM read bandwidth of plain non-temporal 16-byte
//     loads over a buffer far larger than the Infinity Cache;
//   * lds_fill_kernel: the decode's page-copy pattern without the products:
//     72 KiB blocks moved HBM -> LDS with global_load_lds_dwordx4, double
//     buffered with one barrier per block, which bounds how fast a CU can
//     fill its LDS with pages;
//   * lds_operand_kernel: LDS reads of MFMA operands, alone and feeding
//     32x32x16 MFMAs, at the decode's one KiB per wave per MFMA;
//   * block_write_kernel: one contiguous block written per workgroup, the
//     way the decode writes its split partials.
// None of these is on the decode path; they calibrate its measurements.
#include "../../include/mla_ceiling.h"
#include "decode_device.h"

namespace mla {

template <int KIND, int NACC>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* sink) {
  // operands depend on the lane so the compiler cannot fold them
  const int lane = threadIdx.x & 63;
  u32x4 ua = {0x3f803f80u ^ (uint32_t)lane, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  u32x4 ub = {0x3f803f80u, 0x3f803f80u ^ (uint32_t)threadIdx.x, 0x3f803f80u, 0x3f803f80u};
  const bf16x8 a = __builtin_bit_cast(bf16x8, ua), b = __builtin_bit_cast(bf16x8, ub);
  float total = 0.f;
  if constexpr (KIND == 0) {
    // distinct starting values: with identical ones the compiler shuffled
    // the loop-carried accumulators between registers on every iteration
    f32x4 acc[NACC];
#pragma unroll
    for (int k = 0; k < NACC; ++k) acc[k] = f32x4{(float)(lane + k), 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int k = 0; k < NACC; ++k) acc[k] = mfma16(a, b, acc[k]);
    }
#pragma unroll
    for (int k = 0; k < NACC; ++k) total += acc[k][0] + acc[k][3];
  } else {
    f32x16 acc[NACC];
#pragma unroll
    for (int k = 0; k < NACC; ++k)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[k][r] = r == 0 ? (float)(lane + k) : 0.f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int k = 0; k < NACC; ++k) acc[k] = mfma32(a, b, acc[k]);
    }
#pragma unroll
    for (int k = 0; k < NACC; ++k) total += acc[k][0] + acc[k][15];
  }
  sink[blockIdx.x * blockDim.x + threadIdx.x] = total;
}

// Grid-stride 16-byte non-temporal loads; each thread folds what it reads
// into one word so that the loads stay live.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* src, size_t n16,
                                                          uint32_t* sink) {
  uint32_t x = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i);
    const u32x4 v1 = __builtin_nontemporal_load(src + i + stride);
    const u32x4 v2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 v3 = __builtin_nontemporal_load(src + i + 3 * stride);
    x ^= v0[0] ^ v0[1] ^ v0[2] ^ v0[3] ^ v1[0] ^ v1[1] ^ v1[2] ^ v1[3];
    x ^= v2[0] ^ v2[1] ^ v2[2] ^ v2[3] ^ v3[0] ^ v3[1] ^ v3[2] ^ v3[3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = x;
}

// Workgroup w copies blocks w, w + grid, ... (72 KiB each) into two LDS
// buffers in turn, each wave issuing every NW-th 1 KiB copy, with one wait
// and one barrier per block: the decode's copy loop with nothing else in it.
template <int NW>
__global__ __launch_bounds__(64 * NW) void lds_fill_kernel(const char* src, int nblocks,
                                                           uint32_t* sink) {
  constexpr int BLK = 72 * 1024, NDMA = 72 / NW;
  __shared__ __attribute__((aligned(1024))) char lds[2 * BLK];
  const uint32_t lds0 = (uint32_t)(uintptr_t)LDS_PTR(char, lds);
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  auto issue = [&](int blk, int buf) {
    const char* base = uniform_ptr(src + (size_t)blk * BLK);
#pragma unroll
    for (int t = 0; t < NDMA; ++t) {
      const int i = wave + NW * t;
      dma16(lds0 + buf * BLK + 1024 * i, base, 1024 * i + 16 * lane);
    }
  };
  int cur = 0;
  int blk = blockIdx.x;
  if (blk < nblocks) issue(blk, 0);
  for (; blk < nblocks; blk += gridDim.x) {
    wait_vm<0>();
    barrier();
    if (blk + (int)gridDim.x < nblocks) issue(blk + gridDim.x, cur ^ 1);
    cur ^= 1;
  }
  wait_vm<0>();
  barrier();
  // one word of the last buffer keeps the copies observable
  if (threadIdx.x == 0) sink[blockIdx.x] = *(const __attribute__((address_space(3))) uint32_t*)(
      LDS_PTR(char, lds) + cur * BLK);
}

// LDS operand rate, alone and feeding 32x32x16 MFMAs: every wave reads
// 1 KiB of LDS per step (MODE 0, 1: one ds_read_b128 per lane; MODE 2, 3:
// two transposed ds_read_b64_tr_b16 per lane), in MODE 1 and 2 the read
// being the A operand of one MFMA into one of four accumulators. MODE 1 is
// the shape of the decode's score steps, MODE 2 of its P V steps: 4 waves
// of a CU reading the same bytes, each for its own 32 query rows. MODE 4
// and 5 are MODE 1 and 2 with each operand requested eight steps before
// its MFMA, across loop iterations.
template <int MODE, int NW>
__global__ __launch_bounds__(64 * NW) void lds_operand_kernel(int iters, float* sink) {
  constexpr int BYTES = 64 * 1024;
  __shared__ __attribute__((aligned(1024))) char lds[BYTES];
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < BYTES / 4; i += 64 * NW)
    *LDS_PTR(uint32_t, lds + 4 * i) = 0x3f803f80u ^ (uint32_t)(i & 0x00ff00ffu);
  __syncthreads();
  u32x4 ub = {0x3f803f80u, 0x3f803f80u ^ (uint32_t)lane, 0x3f803f80u, 0x3f803f80u};
  const bf16x8 b = __builtin_bit_cast(bf16x8, ub);
  f32x16 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[k][r] = r == 0 ? (float)(lane + k) : 0.f;
  u32x4 x = {0u, 0u, 0u, 0u};
  if constexpr (MODE >= 4) {
    // software pipelined: the operand of step n + D is requested before the
    // MFMA of step n, across iterations (D = 8 steps; mode 4 one b128 read
    // per step, mode 5 two transposed b64 reads)
    constexpr int D = 8;
    auto addr = [&](int n) { return ((n & 63) * 1024) + (MODE == 4 ? 16 : 8) * lane; };
    auto fetch = [&](int n) -> bf16x8 {
      if constexpr (MODE == 4) {
        return *LDS_PTR(bf16x8, lds + addr(n));
      } else {
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)(LDS_PTR(char, lds) + addr(n)));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)(LDS_PTR(char, lds) + addr(n) + 512));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
    bf16x8 ring[D];
#pragma unroll
    for (int k = 0; k < D; ++k) ring[k] = fetch(k);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        const bf16x8 a = ring[st % D];
        ring[st % D] = fetch(16 * i + st + D);
        acc[st & 3] = mfma32(a, b, acc[st & 3]);
        __builtin_amdgcn_sched_barrier(0);  // keeps each read in its step
      }
    }
#pragma unroll
    for (int k = 0; k < D; ++k) x ^= __builtin_bit_cast(u32x4, ring[k]);
  } else
  for (int i = 0; i < iters; ++i) {
    const int base = (i & 3) * 16384;
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      bf16x8 a;
      if constexpr (MODE == 0 || MODE == 1) {
        a = *LDS_PTR(bf16x8, lds + base + st * 1024 + 16 * lane);
      } else {
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)(LDS_PTR(char, lds) + base + st * 1024 + 8 * lane));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)(LDS_PTR(char, lds) + base + st * 1024 + 512 + 8 * lane));
        a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      if constexpr (MODE == 1 || MODE == 2)
        acc[st & 3] = mfma32(a, b, acc[st & 3]);
      else
        x ^= __builtin_bit_cast(u32x4, a);
    }
  }
  float total = __builtin_bit_cast(float, x[0] ^ x[1] ^ x[2] ^ x[3]);
#pragma unroll
  for (int k = 0; k < 4; ++k) total += acc[k][0] + acc[k][15];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = total;
}

// Workgroup w writes `block` bytes at dst + w * stride, each wave 1 KiB per
// store instruction (16 bytes per lane, lanes consecutive): the decode's
// split partials leave this way, 256 KiB per workgroup.
__global__ __launch_bounds__(256) void block_write_kernel(char* dst, size_t block, size_t stride) {
  const u32x4 v = {threadIdx.x, blockIdx.x, 0x3f800000u, 0u};
  char* base = dst + blockIdx.x * stride;
  for (size_t off = 16 * threadIdx.x; off + 16 <= block; off += 16 * 256)
    *(u32x4*)(base + off) = v;
}

}  // namespace mla

extern "C" {

int mla_ceiling_mfma(int32_t kind, int32_t accumulators, int32_t waves_per_simd, int32_t iters,
                     int32_t grid, float* sink, hipStream_t stream) {
  if (!sink) return MLA_CEIL_ERR_ARG;
  if (iters < 1 || grid < 1 || (waves_per_simd != 1 && waves_per_simd != 2))
    return MLA_CEIL_ERR_ARG;
  const dim3 block(256);
  const dim3 g(grid * waves_per_simd);
#define MFMA_CASE(K, N)                                                                    \
  if (kind == K && accumulators == N) {                                                    \
    hipLaunchKernelGGL((mla::mfma_loop_kernel<K, N>), g, block, 0, stream, iters, sink);    \
    return hipGetLastError() == hipSuccess ? 0 : MLA_CEIL_ERR_HIP;                         \
  }
  MFMA_CASE(0, 4)
  MFMA_CASE(0, 8)
  MFMA_CASE(1, 2)
  MFMA_CASE(1, 4)
#undef MFMA_CASE
  return MLA_CEIL_ERR_ARG;
}

int mla_ceiling_stream_read(const void* src, size_t bytes, int32_t grid, uint32_t* sink,
                            hipStream_t stream) {
  if (!src || !sink || grid < 1 || bytes < 16 || (bytes & 15) || ((uintptr_t)src & 15))
    return MLA_CEIL_ERR_ARG;
  hipLaunchKernelGGL(mla::stream_read_kernel, dim3(grid), dim3(256), 0, stream,
                     (const mla::u32x4*)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : MLA_CEIL_ERR_HIP;
}

int mla_ceiling_lds_fill(const void* src, size_t bytes, int32_t waves, int32_t grid,
                         uint32_t* sink, hipStream_t stream) {
  const size_t nb = bytes / (72 * 1024);  // whole 72 KiB blocks only
  if (!src || !sink || nb < 1 || nb > 0x7fffffff || grid < 1 || ((uintptr_t)src & 15))
    return MLA_CEIL_ERR_ARG;
  const int nblocks = (int)nb;
  if (waves == 4)
    hipLaunchKernelGGL(mla::lds_fill_kernel<4>, dim3(grid), dim3(256), 0, stream,
                       (const char*)src, nblocks, sink);
  else if (waves == 8)
    hipLaunchKernelGGL(mla::lds_fill_kernel<8>, dim3(grid), dim3(512), 0, stream,
                       (const char*)src, nblocks, sink);
  else
    return MLA_CEIL_ERR_ARG;
  return hipGetLastError() == hipSuccess ? 0 : MLA_CEIL_ERR_HIP;
}

int mla_ceiling_lds_operand(int32_t mode, int32_t waves, int32_t iters, int32_t grid, float* sink,
                            hipStream_t stream) {
  if (!sink || iters < 1 || grid < 1) return MLA_CEIL_ERR_ARG;
#define LDS_CASE(M, W)                                                                       \
  if (mode == M && waves == W) {                                                             \
    hipLaunchKernelGGL((mla::lds_operand_kernel<M, W>), dim3(grid), dim3(64 * W), 0, stream,  \
                       iters, sink);                                                         \
    return hipGetLastError() == hipSuccess ? 0 : MLA_CEIL_ERR_HIP;                           \
  }
  LDS_CASE(0, 4)
  LDS_CASE(1, 4)
  LDS_CASE(2, 4)
  LDS_CASE(3, 4)
  LDS_CASE(0, 8)
  LDS_CASE(1, 8)
  LDS_CASE(2, 8)
  LDS_CASE(3, 8)
  LDS_CASE(4, 4)
  LDS_CASE(5, 4)
  LDS_CASE(4, 8)
  LDS_CASE(5, 8)
#undef LDS_CASE
  return MLA_CEIL_ERR_ARG;
}

int mla_ceiling_block_write(void* dst, size_t block_bytes, size_t stride_bytes, int32_t grid,
                            hipStream_t stream) {
  if (!dst || grid < 1 || block_bytes < 16 || (block_bytes & 15) || stride_bytes < block_bytes ||
      (stride_bytes & 15) || ((uintptr_t)dst & 15))
    return MLA_CEIL_ERR_ARG;
  hipLaunchKernelGGL(mla::block_write_kernel, dim3(grid), dim3(256), 0, stream, (char*)dst,
                     block_bytes, stride_bytes);
  return hipGetLastError() == hipSuccess ? 0 : MLA_CEIL_ERR_HIP;
}

}  // extern "C"
