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

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t st) {
  const long long tokens = (long long)a.B * a.T;
  if (tokens == 0) return hipSuccess;
  if (tokens > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)tokens), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace mla
