// The two small kernels around the fused decode: the split-KV plan and the
// log-sum-exp merge of split results.
#include "device_common.h"
#include "kernels.h"
#include "schedule.h"

namespace mla {

constexpr int PLAN_THREADS = 1024;

// Inclusive scan of one value per thread over the block; *total gets the
// sum of all values. Each wave scans its 64 values with lane shuffles, wave
// 0 scans the 16 wave totals: three barriers instead of two per doubling
// step over the whole block.
constexpr int PLAN_WAVES = PLAN_THREADS / 64;

__device__ int block_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  if (wv == 0) {
    int t = lane < PLAN_WAVES ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < PLAN_WAVES; off <<= 1) {
      const int y = __shfl_up(t, off);
      if (lane >= off) t += y;
    }
    if (lane < PLAN_WAVES) wsum[lane] = t;
  }
  __syncthreads();
  const int r = x + (wv > 0 ? wsum[wv - 1] : 0);
  *total = wsum[PLAN_WAVES - 1];
  __syncthreads();  // wsum is reused by the next scan
  return r;
}

// One workgroup. Writes the unit prefix (B + 1 entries after the W worker
// records), every worker record, and the exclusive prefix of partial slots
// (B + 1 entries).
__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(const int32_t* seqlens, int B, int W,
                                                           int32_t* meta, int32_t* slots) {
  __shared__ int buf[PLAN_WAVES];
  const int tid = threadIdx.x;
  int32_t* prefix = meta + (size_t)W * sched::REC;

  int carry = 0, total = 0;
  if (tid == 0) prefix[0] = 0;
  for (int base = 0; base < B; base += PLAN_THREADS) {
    const int b = base + tid;
    const int v = b < B ? sched::seq_units(seqlens[b]) : 0;
    const int inc = block_scan(v, buf, &total);
    if (b < B) prefix[b + 1] = carry + inc;
    carry += total;
  }
  __threadfence_block();
  __syncthreads();

  for (int w = tid; w < W; w += PLAN_THREADS)
    sched::worker_record(w, W, prefix, seqlens, B, meta + (size_t)w * sched::REC);

  carry = 0;
  for (int base = 0; base < B; base += PLAN_THREADS) {
    const int b = base + tid;
    const int v = b < B ? sched::seq_slots(b, W, prefix, seqlens, B) : 0;
    const int inc = block_scan(v, buf, &total);
    if (b < B) slots[b] = carry + inc - v;
    carry += total;
  }
  if (tid == 0) slots[B] = carry;
}

hipError_t launch_plan_kernel(const int32_t* seqlens, int B, int W, int32_t* meta,
                              int32_t* slots, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, st, seqlens, B, W, meta, slots);
  return hipGetLastError();
}

// Merge the partials of one (sequence, row): lse = m + ln sum exp(lse_i - m),
// out = sum exp(lse_i - lse) o_i. Grid (R, B); 64 threads, 4 columns each.
__global__ __launch_bounds__(64) void combine_kernel(CombineArgs a) {
  const int rho = blockIdx.x, b = blockIdx.y;
  const int s0 = a.slots[b];
  const int ns = a.slots[b + 1] - s0;
  if (ns <= 0) return;
  const float* pl = a.part_lse + (size_t)s0 * a.R + rho;
  float mx = -INFINITY;
  for (int i = 0; i < ns; ++i) mx = fmaxf(mx, pl[(size_t)i * a.R]);
  uint16_t* orow = a.out + ((size_t)b * a.R + rho) * a.DV;
  if (mx == -INFINITY) {
    for (int c = threadIdx.x * 4; c < a.DV; c += 64 * 4) *(u32x2*)(orow + c) = u32x2{0u, 0u};
    if (threadIdx.x == 0) a.lse[(size_t)b * a.R + rho] = -INFINITY;
    return;
  }
  float tot = 0.f;
  for (int i = 0; i < ns; ++i) tot += fast_exp2((pl[(size_t)i * a.R] - mx) * LOG2E);
  const float inv = 1.f / tot;
  for (int c = threadIdx.x * 4; c < a.DV; c += 64 * 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < ns; ++i) {
      const float wgt = fast_exp2((pl[(size_t)i * a.R] - mx) * LOG2E) * inv;
      const f32x4 x = *(const f32x4*)(a.part_o + (((size_t)(s0 + i) * a.R + rho) * a.DV + c));
      acc += wgt * x;
    }
    u32x2 y;
    y[0] = pack_bf16x2(acc[0], acc[1]);
    y[1] = pack_bf16x2(acc[2], acc[3]);
    *(u32x2*)(orow + c) = y;
  }
  if (threadIdx.x == 0) a.lse[(size_t)b * a.R + rho] = mx + __logf(tot);
}

hipError_t launch_combine_kernel(const CombineArgs& a, hipStream_t st) {
  if (a.B <= 0 || a.R <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(a.R, a.B), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace mla
