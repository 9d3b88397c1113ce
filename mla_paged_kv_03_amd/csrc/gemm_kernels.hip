// The dense products around GQLA decode: the group-indexed up-projections
// (GQLA review, "2. Motivation & Problem Statement": W_UK and W_UV are indexed
// by KV group, so one set of weights serves both decode paths). The absorb
// path multiplies each query's no-rope part by W_UK^g^T before attending the
// latent rows and the latent result by W_UV^g after; the GQA path expands the
// latent rows into per-group K = [c W_UK^g, k_rope] and V = c W_UV^g.
//
// One bf16 GEMM kernel serves all three: a TBM x 128 output tile per
// workgroup of 4 waves (TBM = 128, 64 or 32 by problem size; 16 x 16 x 32
// MFMA), K in steps of 64 staged through LDS in two buffers, the next two
// steps' tiles loaded into registers ahead of use. The rope columns, which
// pass through unchanged, are copied by the first column tile of each row
// tile.
#include "device_common.h"
#include "kernels.h"

namespace mla {

namespace {

constexpr int TBN = 128, TBK = 64;
// LDS rows: 64 k (128 bytes) + 16 bytes, so the 16 rows a 16-lane group
// reads start 36 dwords apart and fall on distinct banks; B stored [k][n]:
// 128 n (256 bytes) + 32, so the four rows of a transposed read start 8
// dwords apart.
constexpr int A_PITCH = 144;
constexpr int BNK_PITCH = 144;
constexpr int BKN_PITCH = 288;
constexpr int B_TILE = TBN * BNK_PITCH;    // 18432 = TBK * BKN_PITCH
static_assert(TBK * BKN_PITCH == B_TILE, "both B layouts fill one tile");

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

// A TBM x 128 output tile per workgroup of 4 waves in a WGM x WGN grid; a
// wave owns a WTM x WTN block (MB x NB blocks of 16 x 16): 64 x 64 for
// TBM = 128, 32 x 64 for 64, 32 x 32 for 32. K runs in steps of 64 through
// two LDS buffers; the tiles of the next two steps are in registers or in
// flight while one is multiplied.
template <bool KN, int TBM>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
  constexpr int A_TILE = TBM * A_PITCH;
  constexpr int STAGE = A_TILE + B_TILE;
  constexpr int AC = TBM * 8 / 256;  // 16-byte A chunks per thread per step
  constexpr int WGM = TBM >= 64 ? 2 : 1, WGN = 4 / WGM;
  constexpr int WTM = TBM / WGM, WTN = TBN / WGN;
  constexpr int MB = WTM / 16, NB = WTN / 16;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  lds_char* const lds = LDS_PTR(char, smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Work item L = (tile, z) with z fastest; workgroup b runs on XCD b % 8
  // (round-robin dispatch) and takes item (b % 8) * per_xcd + b / 8, so each
  // XCD walks a contiguous run of items: the problems that read the same A
  // tile (the expansion's groups) run back to back and share its L2.
  const int ntn = p.N / TBN;
  const int per_xcd = gridDim.x >> 3;
  const int64_t item = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int64_t tile = item / p.batches;
  const int z = (int)(item - tile * p.batches);
  if (tile >= (int64_t)((p.M + TBM - 1) / TBM) * ntn) return;
  const int tm = (int)(tile / ntn), tn = (int)(tile - (int64_t)tm * ntn);
  const int m0 = tm * TBM, n0 = tn * TBN;

  // global -> register -> LDS staging
  const uint16_t* a_src[AC];
  const uint16_t* b_src[4];
  uint32_t a_dst[AC], b_dst[4];
#pragma unroll
  for (int i = 0; i < AC; ++i) {
    const int id = tid + 256 * i;
    const int row = id >> 3, ch = id & 7;   // A: TBM rows x 8 chunks
    const int m = min(m0 + row, p.M - 1);   // rows past M repeat the last one, never stored
    a_src[i] = p.a + p.a_batch * z + row_offset(m, p.inner, p.a_outer, p.a_inner) + 8 * ch;
    a_dst[i] = row * A_PITCH + 16 * ch;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = tid + 256 * i;
    if (KN) {
      const int kr = id >> 4, nc = id & 15;  // B [k][n]: 64 rows x 16 chunks
      b_src[i] = p.b + p.b_batch * z + (int64_t)kr * p.ldb + n0 + 8 * nc;
      b_dst[i] = A_TILE + kr * BKN_PITCH + 16 * nc;
    } else {
      const int row = id >> 3, ch = id & 7;  // B [n][k]: 128 rows x 8 chunks
      b_src[i] = p.b + p.b_batch * z + (int64_t)(n0 + row) * p.ldb + 8 * ch;
      b_dst[i] = A_TILE + row * BNK_PITCH + 16 * ch;
    }
  }
  const int64_t b_step = KN ? (int64_t)TBK * p.ldb : TBK;
  struct Stage {
    u32x4 a[AC], b[4];
  };
  auto load = [&](int kt, Stage& r) {
#pragma unroll
    for (int i = 0; i < AC; ++i) r.a[i] = *(const u32x4*)(a_src[i] + (int64_t)kt * TBK);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.b[i] = *(const u32x4*)(b_src[i] + (int64_t)kt * b_step);
  };
  auto store = [&](int buf, const Stage& r) {
#pragma unroll
    for (int i = 0; i < AC; ++i)
      *(__attribute__((address_space(3))) u32x4*)(lds + buf * STAGE + a_dst[i]) = r.a[i];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(__attribute__((address_space(3))) u32x4*)(lds + buf * STAGE + b_dst[i]) = r.b[i];
  };

  // this lane's fragment addresses (bytes within a stage)
  const int l16 = lane & 15, g4 = lane >> 4;
  const int wm = wave % WGM, wn = wave / WGM;
  const uint32_t a_frag = (WTM * wm + l16) * A_PITCH + 8 * g4;
  const uint32_t b_frag = KN ? A_TILE + (4 * g4 + (l16 >> 2)) * BKN_PITCH + 2 * (WTN * wn + 4 * (l16 & 3))
                             : A_TILE + (WTN * wn + l16) * BNK_PITCH + 8 * g4;

  f32x4 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = p.K / TBK;
  Stage r0, r1;
  load(0, r0);
  if (KT > 1) load(1, r1);
  store(0, r0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    // r1 holds step kt + 1 (loaded earlier); step kt + 2 goes into r0
    if (kt + 2 < KT) load(kt + 2, r0);
    const lds_char* st = lds + cur * STAGE;
#pragma unroll
    for (int s = 0; s < TBK / 32; ++s) {
      bf16x8 af[MB], bfr[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        bfr[nb] = KN ? frag_tr(st + b_frag + nb * 32 + 32 * s * BKN_PITCH)
                     : frag_rows(st + b_frag + nb * 16 * BNK_PITCH + 64 * s);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) af[mb] = frag_rows(st + a_frag + mb * 16 * A_PITCH + 64 * s);
      // C^T tile: the B fragment supplies rows (n), the A fragment columns (m)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = mfma16(bfr[nb], af[mb], acc[nb][mb]);
    }
    if (kt + 1 < KT) store(cur ^ 1, r1);
    __syncthreads();
    r1 = r0;
  }

  // lane l holds C[m = .. + l % 16][n = .. + 4 (l / 16) + r], r = 0..3
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = m0 + WTM * wm + 16 * mb + l16;
    if (m >= p.M) continue;
    uint16_t* crow = p.c + p.c_batch * z + row_offset(m, p.inner, p.c_outer, p.c_inner);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = n0 + WTN * wn + 16 * nb + 4 * g4;
      u32x2 x;
      x[0] = pack_bf16x2(acc[nb][mb][0], acc[nb][mb][1]);
      x[1] = pack_bf16x2(acc[nb][mb][2], acc[nb][mb][3]);
      *(u32x2*)(crow + n) = x;
    }
  }
  // the first column tile also copies its rows' 64 rope columns from the A
  // row to the C row (16-byte chunks, 8 per row)
  if (p.rope && tn == 0) {
    for (int id = tid; id < TBM * 8; id += 256) {
      const int m = m0 + (id >> 3), ch = id & 7;
      if (m >= p.M) continue;
      const uint16_t* src = p.a + p.a_batch * z + row_offset(m, p.inner, p.a_outer, p.a_inner) +
                            p.rope_a_off + 8 * ch;
      uint16_t* dst = p.c + p.c_batch * z + row_offset(m, p.inner, p.c_outer, p.c_inner) +
                      p.rope_c_off + 8 * ch;
      *(u32x4*)dst = *(const u32x4*)src;
    }
  }
}

template <int TBM>
hipError_t launch_tbm(const GemmArgs& a, hipStream_t st) {
  const int64_t items = (int64_t)((a.M + TBM - 1) / TBM) * (a.N / TBN) * a.batches;
  const int64_t per_xcd = (items + 7) / 8;
  if (8 * per_xcd > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(8 * per_xcd));
  if (a.b_kn)
    hipLaunchKernelGGL((gemm_kernel<true, TBM>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((gemm_kernel<false, TBM>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.M == 0 || a.batches == 0) return hipSuccess;
  if (a.M < 0 || a.N <= 0 || a.K <= 0 || a.N % TBN || a.K % TBK || a.inner < 1 ||
      a.batches > 65535)
    return hipErrorInvalidValue;
  // smaller row tiles for short problems, so that they still fill the chip
  if (a.M >= 8192) return launch_tbm<128>(a, st);
  if (a.M >= 2048) return launch_tbm<64>(a, st);
  return launch_tbm<32>(a, st);
}

}  // namespace mla
