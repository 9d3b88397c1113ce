// The dense products around GQLA decode: the group-indexed up-projections
// (GQLA review, "2. Motivation & Problem Statement": W_UK and W_UV are indexed
// by KV group, so one set of weights serves both decode paths). The absorb
// path multiplies each query's no-rope part by W_UK^g^T before attending the
// latent rows and the latent result by W_UV^g after; the GQA path expands the
// latent rows into per-group K = [c W_UK^g, k_rope] and V = c W_UV^g.
//
// One bf16 GEMM kernel serves all three: a 128 x 128 output tile per
// workgroup of 4 waves (each 64 x 64 = 4 x 4 blocks of 16 x 16 x 32 MFMA),
// K in steps of 64 staged through LDS in two buffers; the next step's tile
// is loaded into registers while the current one is multiplied.
#include "device_common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int TBM = 128, TBN = 128, TBK = 64;
// LDS rows: 64 k (128 bytes) + 16 bytes, so the 16 rows a 16-lane group
// reads start 36 dwords apart and fall on distinct banks; B stored [k][n]:
// 128 n (256 bytes) + 32, so the four rows of a transposed read start 8
// dwords apart.
constexpr int A_PITCH = 144;
constexpr int BNK_PITCH = 144;
constexpr int BKN_PITCH = 288;
constexpr int A_TILE = TBM * A_PITCH;      // 18432
constexpr int B_TILE = TBN * BNK_PITCH;    // 18432 = TBK * BKN_PITCH
static_assert(TBK * BKN_PITCH == B_TILE, "both B layouts fill one tile");
constexpr int STAGE = A_TILE + B_TILE;

__device__ __forceinline__ int64_t row_offset(int m, int inner, int64_t outer_s, int64_t inner_s) {
  const int o = m / inner;
  return (int64_t)o * outer_s + (int64_t)(m - o * inner) * inner_s;
}

// Both MFMA operands hold, in slot i of lane l, k = 16 (i / 4) + 4 (l / 16) + i % 4
// of their 32-wide K step: the order the transposed LDS read gives for a
// [k][n] operand. An MFMA sums over its slots in any order as long as both
// operands agree, so the [m][k] and [n][k] operands are read in that order
// too (two 8-byte reads at k and k + 16).
__device__ __forceinline__ bf16x8 frag_rows(const lds_char* p) {
  const bf16x4 lo = *(const __attribute__((address_space(3))) bf16x4*)p;
  const bf16x4 hi = *(const __attribute__((address_space(3))) bf16x4*)(p + 32);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 frag_tr(const lds_char* p) {
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 16 * BKN_PITCH));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <bool KN>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  lds_char* const lds = LDS_PTR(char, smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntn = p.N / TBN;
  const int tm = blockIdx.x / ntn, tn = blockIdx.x - tm * ntn;
  const int z = blockIdx.y;
  const int m0 = tm * TBM, n0 = tn * TBN;

  // Global -> register -> LDS staging: 4 16-byte chunks of A and of B per thread.
  const uint16_t* a_src[4];
  const uint16_t* b_src[4];
  uint32_t a_dst[4], b_dst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i;
    const int row = id >> 3, ch = id & 7;   // A: 128 rows x 8 chunks
    const int m = min(m0 + row, p.M - 1);   // rows past M repeat the last one, never stored
    a_src[i] = p.a + p.a_batch * z + row_offset(m, p.inner, p.a_outer, p.a_inner) + 8 * ch;
    a_dst[i] = row * A_PITCH + 16 * ch;
    if (KN) {
      const int kr = id >> 4, nc = id & 15;  // B [k][n]: 64 rows x 16 chunks
      b_src[i] = p.b + p.b_batch * z + (int64_t)kr * p.ldb + n0 + 8 * nc;
      b_dst[i] = A_TILE + kr * BKN_PITCH + 16 * nc;
    } else {
      b_src[i] = p.b + p.b_batch * z + (int64_t)(n0 + row) * p.ldb + 8 * ch;
      b_dst[i] = A_TILE + row * BNK_PITCH + 16 * ch;
    }
  }
  const int64_t b_step = KN ? (int64_t)TBK * p.ldb : TBK;
  u32x4 ra[4], rb[4];
  auto load = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = *(const u32x4*)(a_src[i] + (int64_t)kt * TBK);
      rb[i] = *(const u32x4*)(b_src[i] + (int64_t)kt * b_step);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(__attribute__((address_space(3))) u32x4*)(lds + buf * STAGE + a_dst[i]) = ra[i];
      *(__attribute__((address_space(3))) u32x4*)(lds + buf * STAGE + b_dst[i]) = rb[i];
    }
  };

  // this lane's fragment addresses (bytes within a stage)
  const int wm = wave & 1, wn = wave >> 1;
  const int l16 = lane & 15, g4 = lane >> 4;
  const uint32_t a_frag = (64 * wm + l16) * A_PITCH + 8 * g4;
  const uint32_t b_frag = KN ? A_TILE + (4 * g4 + (l16 >> 2)) * BKN_PITCH + 2 * (64 * wn + 4 * (l16 & 3))
                             : A_TILE + (64 * wn + l16) * BNK_PITCH + 8 * g4;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = p.K / TBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load(kt + 1);
    const lds_char* st = lds + cur * STAGE;
#pragma unroll
    for (int s = 0; s < TBK / 32; ++s) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) af[mb] = frag_rows(st + a_frag + mb * 16 * A_PITCH + 64 * s);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        bfr[nb] = KN ? frag_tr(st + b_frag + nb * 32 + 32 * s * BKN_PITCH)
                     : frag_rows(st + b_frag + nb * 16 * BNK_PITCH + 64 * s);
      // C^T tile: the B fragment supplies rows (n), the A fragment columns (m)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = mfma16(bfr[nb], af[mb], acc[nb][mb]);
    }
    if (kt + 1 < KT) store(cur ^ 1);
    __syncthreads();
  }

  // lane l holds C[m = .. + l % 16][n = .. + 4 (l / 16) + r], r = 0..3
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int m = m0 + 64 * wm + 16 * mb + l16;
    if (m >= p.M) continue;
    uint16_t* crow = p.c + p.c_batch * z + row_offset(m, p.inner, p.c_outer, p.c_inner);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = n0 + 64 * wn + 16 * nb + 4 * g4;
      u32x2 x;
      x[0] = pack_bf16x2(acc[nb][mb][0], acc[nb][mb][1]);
      x[1] = pack_bf16x2(acc[nb][mb][2], acc[nb][mb][3]);
      *(u32x2*)(crow + n) = x;
    }
  }
}

// 8 threads per (row, rep), one 16-byte chunk each.
__global__ __launch_bounds__(256) void copy_cols64_kernel(Cols64Args a) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t unit = id >> 3;
  if (unit >= a.rows * a.reps) return;
  const int ch = (int)(id & 7);
  const int64_t r = unit / a.reps;
  const u32x4 v = *(const u32x4*)(a.src + r * a.src_stride + a.src_off + 8 * ch);
  *(u32x4*)(a.dst + unit * a.dst_stride + a.dst_off + 8 * ch) = v;
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.M == 0 || a.batches == 0) return hipSuccess;
  if (a.M < 0 || a.N <= 0 || a.K <= 0 || a.N % TBN || a.K % TBK || a.inner < 1 ||
      a.batches > 65535)
    return hipErrorInvalidValue;
  const int64_t tiles = (int64_t)((a.M + TBM - 1) / TBM) * (a.N / TBN);
  if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tiles, (unsigned)a.batches);
  if (a.b_kn)
    hipLaunchKernelGGL(gemm_kernel<true>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(gemm_kernel<false>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_copy_cols64(const Cols64Args& a, hipStream_t st) {
  const int64_t threads = a.rows * a.reps * 8;
  if (threads == 0) return hipSuccess;
  const int64_t blocks = (threads + 255) / 256;
  if (a.rows < 0 || a.reps < 1 || blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_cols64_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace mla
