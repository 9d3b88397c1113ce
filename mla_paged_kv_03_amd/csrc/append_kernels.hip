// Paged KV append: the new tokens' cache rows written into their page slots
// through the block table, ahead of the decode that reads them.
#include "device_common.h"
#include "kernels.h"

namespace mla {

// One wave per new token. A token row is `row_bytes` contiguous bytes in
// the source (row t of sequence b) and in the cache (slot p % 64 of page
// block_table[b, p / 64], p = L_b - T + t); each lane moves 16-byte chunks.
// A second tensor (the GQA V cache) uses the same slot.
__global__ __launch_bounds__(64) void kv_append_kernel(AppendArgs a) {
  const int b = blockIdx.x / a.T;
  const int t = blockIdx.x - b * a.T;
  const int p = a.seqlens[b] - a.T + t;
  if (p < 0) return;  // the sequence holds fewer than T tokens: only its last ones exist
  const int page = a.block_table[(size_t)b * a.bt_stride + (p >> 6)];
  if (page < 0 || page >= a.num_pages) return;  // outside the cache: never written
  const size_t src = ((size_t)b * a.T + t) * a.row_bytes;
  const size_t dst = ((size_t)page * 64 + (p & 63)) * a.row_bytes;
  const int chunks = (int)(a.row_bytes >> 4);
  for (int c = threadIdx.x; c < chunks; c += 64) {
    *(u32x4*)(a.dst0 + dst + 16 * (size_t)c) = *(const u32x4*)(a.src0 + src + 16 * (size_t)c);
    if (a.src1) *(u32x4*)(a.dst1 + dst + 16 * (size_t)c) = *(const u32x4*)(a.src1 + src + 16 * (size_t)c);
  }
}

// FP8 quantisation of one 576-wide latent row per wave: amax over the row;
// the scale is the smallest power of two not below the float32 quotient
// amax / 448 (at least 2^-126; 1 for an all-zero row), so x / scale is
// exact, and every code is the E4M3 value nearest (ties to even) to x / scale
// clamped to +-448. A power-of-two scale also keeps the decode exact where
// it multiplies softmax weights by the scale before rounding them to bf16.
// The conversion rounds to nearest even and, without the clamp, would turn
// values past 464 into NaN. Lane l holds 16-byte chunk l (and chunk 64 + l
// for l < 8) of the row.
__global__ __launch_bounds__(64) void quantize_fp8_kernel(QuantArgs a) {
  constexpr int D = 576, CH = D / 8;
  const int r = blockIdx.x;
  const int lane = threadIdx.x;
  int64_t drow = r;
  if (a.block_table) {
    const int b = r / a.T, t = r - b * a.T;
    const int p = a.seqlens[b] - a.T + t;
    if (p < 0) return;
    const int page = a.block_table[(size_t)b * a.bt_stride + (p >> 6)];
    if (page < 0 || page >= a.num_pages) return;
    drow = (int64_t)page * 64 + (p & 63);
  }
  const uint16_t* src = a.src + (int64_t)r * D;
  float x[2][8];
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    if (c < CH) {
      const u32x4 w = *(const u32x4*)(src + 8 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[k][2 * i] = __uint_as_float(w[i] << 16);
        x[k][2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[k][i]));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  float scale = 1.f;
  if (amax > 0.f) {
    const uint32_t r = __float_as_uint(amax / 448.f);
    scale = r < 0x00800000u ? __uint_as_float(0x00800000u)                    // 2^-126
            : (r & 0x007fffffu) == 0 ? __uint_as_float(r)                     // a power of two
                                     : __uint_as_float((r & 0x7f800000u) + 0x00800000u);
  }
  uint8_t* dst = a.codes + drow * D;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    if (c < CH) {
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(x[k][i] / scale, -448.f), 448.f);
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
      *(u32x2*)(dst + 8 * c) = u32x2{(uint32_t)lo, (uint32_t)hi};
    }
  }
  if (lane == 0) a.scales[drow] = scale;
}

hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t st) {
  const long long rows = (long long)a.B * a.T;
  if (rows == 0) return hipSuccess;
  if (rows > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3((unsigned)rows), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t st) {
  const long long tokens = (long long)a.B * a.T;
  if (tokens == 0) return hipSuccess;
  if (tokens > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)tokens), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace mla
