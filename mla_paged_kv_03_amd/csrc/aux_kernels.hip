// The two small kernels around the fused decode: the split-KV plan and the
// log-sum-exp merge of split results.
#include "device_common.h"
#include "kernels.h"
#include "schedule.h"

namespace mla {

constexpr int PLAN_THREADS = 256;

// Inclusive scan of one value per thread over the block; *total gets the
// sum of all values. Each wave scans its 64 values with lane shuffles, wave
// 0 scans the wave totals: three barriers instead of two per doubling step
// over the whole block.
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

// Batches up to this many sequences keep the unit prefix and the lengths in
// LDS, where the workers' binary searches run; larger ones search them in
// global memory.
constexpr int PLAN_LDS_SEQS = 8192;
// Plans over up to this many workers find each worker's first and last
// sequences through an LDS table filled by the sequences (below).
constexpr int PLAN_LDS_WORKERS = 2048;

// One workgroup. Writes the plan's signature, the unit prefix (B + 1 entries
// after the W worker records), every worker record, and the exclusive prefix
// of partial slots (B + 1 entries): schedule.h's host_plan, in parallel.
__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(const int32_t* seqlens, int B, int W,
                                                           int rows, int G, int DV, int fix,
                                                           int32_t* meta, int32_t* slots) {
  __shared__ int buf[PLAN_WAVES];
  __shared__ int32_t s_prefix[PLAN_LDS_SEQS + 1];
  __shared__ int32_t s_len[PLAN_LDS_SEQS];
  __shared__ int32_t s_pcs[PLAN_LDS_SEQS];       // pieces of each sequence
  __shared__ int32_t s_own[PLAN_LDS_WORKERS];    // sequence where a worker's range starts
  const int tid = threadIdx.x;
  int32_t* prefix = sched::unit_prefix(meta, W);
  const bool in_lds = B <= PLAN_LDS_SEQS;

  // step 1: the batch's cost T, each sequence taken whole: per-thread sums,
  // a wave reduction, one barrier
  __shared__ int s_red[PLAN_WAVES];
  int part = 0;
  for (int b = tid; b < B; b += PLAN_THREADS) {
    const int L = seqlens[b];
    part += sched::seq_cost(L, fix);
    if (in_lds) s_len[b] = L;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
  if ((tid & 63) == 0) s_red[tid >> 6] = part;
  __syncthreads();
  int T = 0, total = 0;
#pragma unroll
  for (int i = 0; i < PLAN_WAVES; ++i) T += s_red[i];
  if (tid == 0) {
    sched::write_header(meta, W, B, rows, G, DV, fix, T);
    prefix[0] = 0;
    s_prefix[0] = 0;
  }
  // (each thread reads back only the lengths it stored itself until the
  // scan's barriers)
  const int32_t* len = in_lds ? s_len : seqlens;
  // step 2: the line of blocks and its prefix
  int carry = 0;
  for (int base = 0; base < B; base += PLAN_THREADS) {
    const int b = base + tid;
    int v = 0;
    if (b < B) {
      const int n = sched::seq_pieces(len[b], fix, T, W);
      v = sched::seq_pages(len[b]) + fix * n;  // seq_units
      if (in_lds) s_pcs[b] = n;
    }
    const int inc = block_scan(v, buf, &total);
    if (b < B) {
      prefix[b + 1] = carry + inc;
      if (in_lds) s_prefix[b + 1] = carry + inc;
    }
    carry += total;
  }
  __threadfence_block();
  __syncthreads();
  const int32_t* pre = in_lds ? s_prefix : prefix;

  if (in_lds && W <= PLAN_LDS_WORKERS) {
    // Each sequence marks the workers whose range starts among its units
    // (the unit prefix rises strictly, so every worker start has exactly
    // one owner); a worker's last sequence is the owner of its last unit,
    // which the next worker's start gives. The same values as worker_record's
    // binary searches, without their chains of dependent LDS reads.
    const int32_t C = pre[B];
    const int chunk = sched::chunk_units(C, W, fix);
    for (int b = tid; b < B; b += PLAN_THREADS) {
      const int w0 = (pre[b] + chunk - 1) / chunk;
      const int w1 = min((pre[b + 1] + chunk - 1) / chunk, W);
      for (int w = w0; w < w1; ++w) s_own[w] = b;
    }
    __syncthreads();
    for (int w = tid; w < W; w += PLAN_THREADS) {
      int32_t* rec = sched::records(meta) + (size_t)w * sched::REC;
      const int64_t lo = (int64_t)w * chunk;
      if (lo >= C) {
        rec[sched::R_B_START] = 0; rec[sched::R_P_START] = 0; rec[sched::R_B_END] = -1;
        rec[sched::R_P_END] = 0; rec[sched::R_SPLIT0] = 0; rec[sched::R_OWNS_FIRST] = 0;
        rec[sched::R_LO] = C; rec[sched::R_HI] = C;
        continue;
      }
      const int64_t hi = lo + chunk < C ? lo + chunk : C;
      const int bs = s_own[w];
      int be = B - 1;
      if (hi < C) {  // worker w + 1 starts at hi
        const int b1 = s_own[w + 1];
        be = pre[b1] < hi ? b1 : b1 - 1;
      }
      sched::record_of(w, chunk, lo, hi, bs, be, sched::seq_pages(len[bs]), s_pcs[bs],
                       sched::seq_pages(len[be]), s_pcs[be], pre, fix, rec);
    }
  } else {
    for (int w = tid; w < W; w += PLAN_THREADS)
      sched::worker_record(w, W, pre, len, B, fix, T,
                           sched::records(meta) + (size_t)w * sched::REC);
  }

  carry = 0;
  for (int base = 0; base < B; base += PLAN_THREADS) {
    const int b = base + tid;
    const int v = b < B ? sched::seq_slots(b, W, pre, len, B, fix) : 0;
    const int inc = block_scan(v, buf, &total);
    if (b < B) slots[b] = carry + inc - v;
    carry += total;
  }
  if (tid == 0) slots[B] = carry;
}

hipError_t launch_plan_kernel(const int32_t* seqlens, int B, int W, int rows, int G, int DV,
                              int fix, int32_t* meta, int32_t* slots, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, st, seqlens, B, W, rows, G, DV,
                     fix, meta, slots);
  return hipGetLastError();
}

// Merge the partials of one (sequence, row): lse = m + ln sum exp(lse_i - m),
// out = sum exp(lse_i - lse) o_i. One wave per row, four rows per
// workgroup; grid (ceil(R / 4), B, Z). Lane i holds item i's lse (the max
// and sum are wave reductions); lane l owns columns 4l + 256k, k < NK. The
// first two items' rows load with the lse values, later ones U at a time,
// so independent loads are in flight together: two in the one-pass merge
// of a few partials, which keeps the registers low enough for eight waves
// per SIMD, four where there are many.
//
// Items: level 0 merges every partial of the sequence. A sequence spread
// over many workgroups (one long sequence in a small batch) has up to one
// partial per worker, too many for one wave to walk in order, so the merge
// then takes two launches: level 1 (z = blockIdx.z) merges the z-th chunk of
// ceil(n / Z) consecutive partials into the chunk's first slot, level 2
// merges the chunks' results. Both orders are fixed, so results do not
// depend on timing.
constexpr int COMBINE_ROWS = 4;

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum64(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

template <int NK, int U>
__global__ __launch_bounds__(64 * COMBINE_ROWS) void combine_kernel(CombineArgs a) {
  const int lane = threadIdx.x & 63;
  const int rho = blockIdx.x * COMBINE_ROWS + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (rho >= a.R) return;
  // The sequence's slot range (b < B: inside the B + 1 entries whatever
  // the plan) and, inside a decode call, the plan's signature, all loaded
  // before any of them is tested so that they share one memory round trip.
  // The slot prefix must come from a plan made for this call's geometry,
  // the one the decode kernel checked (else the slots may lie past the
  // workspace, or hold no partials of this call).
  const int s0 = a.slots[b];
  const int s1 = a.slots[b + 1];
  if (a.meta) {
    const int32_t* h = a.meta;
    const int32_t h_magic = h[sched::H_MAGIC], h_w = h[sched::H_W], h_b = h[sched::H_B],
                  h_rows = h[sched::H_ROWS], h_g = h[sched::H_G], h_dv = h[sched::H_DV];
    // bitwise, not short-circuit: no load waits for another's comparison
    if ((h_magic != sched::PLAN_MAGIC) | (h_w != a.W) | (h_b != a.B) | (h_rows != a.R) |
        (h_g != a.G) | (h_dv != a.DV))
      return;
  }
  const int ns = s1 - s0;
  if (ns <= 0) return;
  // this wave's items: slots s0 + first + i * stride, i < n
  int first = 0, stride = 1, n = ns;
  if (a.level != 0) {
    const int c = (ns + a.Z - 1) / a.Z;  // chunk length
    if (a.level == 1) {
      first = blockIdx.z * c;
      n = min(c, ns - first);
      if (c <= 1 || n <= 0) return;  // c = 1: the partials are the chunks' results
    } else if (c > 1) {
      stride = c;
      n = (ns + c - 1) / c;
    }
  }
  const bool to_out = a.level != 1;  // else a chunk result
  const size_t row = (size_t)(s0 + first) * a.R + rho;
  const float* po = a.part_o + row * a.DV;
  const float* pl = a.part_lse + row;
  const size_t ostride = (size_t)stride * a.R * a.DV, lstride = (size_t)stride * a.R;
  auto load = [&](int i, int k) -> f32x4 {
    const int c = lane * 4 + 256 * k;
    return c < a.DV ? *(const f32x4*)(po + (size_t)i * ostride + c) : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // the first two items' rows are loaded together with the lse values
  // rather than after the weights are known (one memory round trip less)
  f32x4 y[2][NK];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int k = 0; k < NK; ++k) y[u][k] = u < n ? load(u, k) : f32x4{0.f, 0.f, 0.f, 0.f};
  // lane i (and i + 64, ...) holds item i's lse
  const float mine = lane < n ? pl[(size_t)lane * lstride] : -INFINITY;
  float mx = mine;
  for (int i = lane + 64; i < n; i += 64) mx = fmaxf(mx, pl[(size_t)i * lstride]);
  mx = wave_max64(mx);
  if (mx == -INFINITY) {
    // no key at all: out = 0, lse = -inf (also as a chunk's result)
    if (to_out) {
      uint16_t* orow = a.out + ((size_t)b * a.R + rho) * a.DV;
      for (int c = lane * 4; c < a.DV; c += 64 * 4) *(u32x2*)(orow + c) = u32x2{0u, 0u};
      if (lane == 0) a.lse[(size_t)b * a.R + rho] = -INFINITY;
    } else {
      float* crow = a.chunk_o + row * a.DV;
      for (int c = lane * 4; c < a.DV; c += 64 * 4) *(f32x4*)(crow + c) = f32x4{0.f, 0.f, 0.f, 0.f};
      if (lane == 0) a.chunk_lse[row] = -INFINITY;
    }
    return;
  }
  float tot = lane < n ? fast_exp2((mine - mx) * LOG2E) : 0.f;
  for (int i = lane + 64; i < n; i += 64) tot += fast_exp2((pl[(size_t)i * lstride] - mx) * LOG2E);
  tot = wave_sum64(tot);
  const float inv = 1.f / tot;
  const float myw = lane < n ? fast_exp2((mine - mx) * LOG2E) * inv : 0.f;
  auto weight = [&](int i) -> float {
    return i < 64 ? __shfl(myw, i) : fast_exp2((pl[(size_t)i * lstride] - mx) * LOG2E) * inv;
  };
  f32x4 acc[NK];
  {
    const float w0 = weight(0), w1 = n > 1 ? weight(1) : 0.f;
#pragma unroll
    for (int k = 0; k < NK; ++k) acc[k] = w0 * y[0][k] + w1 * y[1][k];
  }
  // the rest U at a time, their loads in flight together
  for (int i = 2; i < n; i += U) {
    f32x4 x[U][NK];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < NK; ++k) x[u][k] = i + u < n ? load(i + u, k) : f32x4{0.f, 0.f, 0.f, 0.f};
    float w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = i + u < n ? weight(i + u) : 0.f;
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
      for (int u = 0; u < U; ++u) acc[k] += w[u] * x[u][k];
  }
  const float lse_v = mx + __logf(tot);
  if (to_out) {
    uint16_t* orow = a.out + ((size_t)b * a.R + rho) * a.DV;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int c = lane * 4 + 256 * k;
      if (c < a.DV) {
        u32x2 z;
        z[0] = pack_bf16x2(acc[k][0], acc[k][1]);
        z[1] = pack_bf16x2(acc[k][2], acc[k][3]);
        *(u32x2*)(orow + c) = z;
      }
    }
    if (lane == 0) a.lse[(size_t)b * a.R + rho] = lse_v;
  } else {
    // over the chunk's first item, whose row this wave has already read
    float* crow = a.chunk_o + row * a.DV;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int c = lane * 4 + 256 * k;
      if (c < a.DV) *(f32x4*)(crow + c) = acc[k];
    }
    if (lane == 0) a.chunk_lse[row] = lse_v;
  }
}

template <int NK>
static void launch_combine_nk(CombineArgs a, hipStream_t st) {
  const dim3 block(64 * COMBINE_ROWS);
  const unsigned gx = (a.R + COMBINE_ROWS - 1) / COMBINE_ROWS;
  if (a.Z <= 1) {
    a.level = 0;
    if (a.wide)
      hipLaunchKernelGGL((combine_kernel<NK, 4>), dim3(gx, a.B), block, 0, st, a);
    else
      hipLaunchKernelGGL((combine_kernel<NK, 2>), dim3(gx, a.B), block, 0, st, a);
    return;
  }
  a.level = 1;
  hipLaunchKernelGGL((combine_kernel<NK, 4>), dim3(gx, a.B, a.Z), block, 0, st, a);
  a.level = 2;
  hipLaunchKernelGGL((combine_kernel<NK, 4>), dim3(gx, a.B), block, 0, st, a);
}

hipError_t launch_combine_kernel(const CombineArgs& a, hipStream_t st) {
  if (a.B <= 0 || a.R <= 0) return hipSuccess;
  if (a.DV > 1024 || a.B > 65535 || a.Z > 65535) return hipErrorInvalidValue;
  if (a.Z > 1 && (!a.chunk_o || !a.chunk_lse)) return hipErrorInvalidValue;
  const int nk = (a.DV + 255) / 256;
  switch (nk) {
    case 1: launch_combine_nk<1>(a, st); break;
    case 2: launch_combine_nk<2>(a, st); break;
    default: launch_combine_nk<4>(a, st); break;
  }
  return hipGetLastError();
}

// Check of the decode calls' device-side preconditions, one workgroup: every
// thread scans a strided share of the (sequence, page) pairs, a length that
// the block table cannot hold counting as page -1 of its sequence. The
// workgroup reduces the violation count and the smallest linear index
// b * (max_pages + 1) + (j + 1) and one thread stores both, so status needs
// no initialisation. Block-table entries are read only for pages a valid
// length uses.
constexpr int CHECK_THREADS = 1024;

__global__ __launch_bounds__(CHECK_THREADS) void check_pages_kernel(
    const int32_t* block_table, const int32_t* seqlens, int B, int num_pages, int max_pages,
    int bt_stride, int32_t* status) {
  __shared__ int s_count[CHECK_THREADS / 64];
  __shared__ int64_t s_first[CHECK_THREADS / 64];
  const int64_t per_seq = (int64_t)max_pages + 1;
  const int64_t n = (int64_t)B * per_seq;
  int count = 0;
  int64_t first = INT64_MAX;
  for (int64_t i = threadIdx.x; i < n; i += CHECK_THREADS) {
    const int b = (int)(i / per_seq);
    const int j = (int)(i - (int64_t)b * per_seq) - 1;  // -1: the length itself
    const int L = seqlens[b];
    const bool len_ok = L >= 0 && (int64_t)L <= 64 * (int64_t)max_pages;
    bool bad;
    if (j < 0) {
      bad = !len_ok;
    } else {
      bad = false;
      if (len_ok && j < (L + 63) / 64) {
        const int page = block_table[(size_t)b * bt_stride + j];
        bad = page < 0 || page >= num_pages;
      }
    }
    if (bad) {
      ++count;
      first = first < i ? first : i;
    }
  }
  // wave reductions, then one value per wave through LDS
  for (int off = 32; off > 0; off >>= 1) {
    count += __shfl_xor(count, off);
    const int64_t o = __shfl_xor(first, off);
    first = first < o ? first : o;
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) {
    s_count[wv] = count;
    s_first[wv] = first;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int c = 0;
    int64_t f = INT64_MAX;
    for (int w = 0; w < CHECK_THREADS / 64; ++w) {
      c += s_count[w];
      f = f < s_first[w] ? f : s_first[w];
    }
    status[0] = c;
    if (f == INT64_MAX) {
      status[1] = -1;
      status[2] = 0;
      status[3] = 0;
    } else {
      const int b = (int)(f / per_seq), j = (int)(f % per_seq) - 1;
      status[1] = b;
      status[2] = j;
      status[3] = j < 0 ? seqlens[b] : block_table[(size_t)b * bt_stride + j];
    }
  }
}

hipError_t launch_check_pages(const int32_t* block_table, const int32_t* seqlens, int B,
                              int num_pages, int max_pages, int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(check_pages_kernel, dim3(1), dim3(CHECK_THREADS), 0, st, block_table, seqlens,
                     B, num_pages, max_pages, max_pages, status);
  return hipGetLastError();
}

// Check of an FP8 cache's per-token scales, one workgroup: a scale passes
// when it is a positive normal power of two (sign 0, exponent field 1..254,
// mantissa field 0), the scales mla_kv_quantize_fp8 writes and the ones the
// 64-row decode dequantises to bf16 exactly. The workgroup counts the others
// and keeps the smallest index among them; one thread stores [count, index
// low word, index high word, the scale's bits], so the status needs no
// initialisation.
__global__ __launch_bounds__(CHECK_THREADS) void check_fp8_scales_kernel(const uint32_t* bits,
                                                                         int64_t n,
                                                                         int32_t* status) {
  __shared__ int s_count[CHECK_THREADS / 64];
  __shared__ int64_t s_first[CHECK_THREADS / 64];
  int count = 0;
  int64_t first = INT64_MAX;
  for (int64_t i = threadIdx.x; i < n; i += CHECK_THREADS) {
    const uint32_t u = bits[i];
    const uint32_t e = (u >> 23) & 0xffu;
    const bool ok = (u >> 31) == 0u && e >= 1u && e <= 254u && (u & 0x7fffffu) == 0u;
    if (!ok) {
      ++count;
      first = first < i ? first : i;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    count += __shfl_xor(count, off);
    const int64_t o = __shfl_xor(first, off);
    first = first < o ? first : o;
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) {
    s_count[wv] = count;
    s_first[wv] = first;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int c = 0;
    int64_t f = INT64_MAX;
    for (int w = 0; w < CHECK_THREADS / 64; ++w) {
      c += s_count[w];
      f = f < s_first[w] ? f : s_first[w];
    }
    status[0] = c;
    if (f == INT64_MAX) f = -1;
    status[1] = (int32_t)(uint32_t)(uint64_t)f;
    status[2] = (int32_t)(uint32_t)((uint64_t)f >> 32);
    status[3] = f < 0 ? 0 : (int32_t)bits[f];
  }
}

hipError_t launch_check_fp8_scales(const float* scales, int64_t n, int32_t* status,
                                   hipStream_t st) {
  hipLaunchKernelGGL(check_fp8_scales_kernel, dim3(1), dim3(CHECK_THREADS), 0, st,
                     (const uint32_t*)scales, n, status);
  return hipGetLastError();
}

}  // namespace mla
