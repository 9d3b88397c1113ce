// GQLA's cache expansion, the GQA path's K and V pages from the latent
// rows (GQLA review, "2. Motivation & Problem Statement": the up-projections
// are indexed by KV group): for every latent row m and group g,
//     C[m, g, 0:128] = A[m, 0:512] . W_g            (W_g: 512 x 128)
// and, for K, C[m, g, 128:192] = A[m, 512:576] (the shared rope columns).
//
// The product has the shape of the decode kernel's score product with the
// roles renamed: latent rows for keys, the 128 weight columns of a group for
// query rows, the 512 latent columns for the head dimension. A workgroup of
// eight waves serves two groups: waves 0-3 hold group 2p's weights in
// registers (each wave 32 columns, 128 VGPRs), waves 4-7 group 2p + 1's, and
// all eight stream 64-row tiles of latent rows HBM -> LDS in the decode page
// layout (rows of 1152 bytes, 16-byte chunk c of row r at c ^ (r & 7)), two
// buffers, the next tile in flight while one is multiplied. Each tile thus
// crosses into a CU once per pair of groups, and each SIMD runs two waves.
// A tile's outputs are staged through its own buffer once the products are
// done, so that every store writes whole 256-byte rows.
//
// Work: the group pairs' workgroups of one slice of rows get ids congruent
// mod 8, so they run on one XCD (round-robin dispatch) and read the slice's
// tiles through the same L2.
#include "decode_device.h"

namespace mla {

namespace {

constexpr int EX_ROWS = 64;                   // latent rows per tile
constexpr int EX_PITCH = 1152;                // bytes per latent row (512 + 64 bf16)
constexpr int EX_TILE = EX_ROWS * EX_PITCH;   // 72 KiB
constexpr int EX_DC = 512, EX_N = 128;        // latent width, columns per group
constexpr int EX_WPITCH = 2 * EX_DC + 16;     // a staged W_g^T row: 512 k + 8 pad (bf16)
constexpr int EX_PF = 3;                      // LDS reads issued this many steps ahead
static_assert(EX_N * EX_WPITCH <= 2 * EX_TILE, "W_g^T is staged in the tile buffers");

__global__ __launch_bounds__(512) void expand_kernel(ExpandArgs p) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * EX_TILE];
  lds_char* const lds_p = LDS_PTR(char, lds);
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds_p;
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int n16 = lane & 15;  // column (MFMA row) within a 16-block, or latent row
  const int g4 = lane >> 4;   // 16-lane group
  const int half = wave >> 2;  // which group of the pair
  const int cw = wave & 3;     // this wave's 32 columns of the group

  // workgroup id -> (group pair, slice of rows); the grid is GP * n_slices
  // and n_slices is a multiple of 8
  const int GP = (p.G + 1) >> 1;
  const int xcd = blockIdx.x & 7, t8 = blockIdx.x >> 3;
  const int gp = t8 % GP;
  const int slice = (t8 / GP) * 8 + xcd;
  const int g = 2 * gp + half;
  const bool live = g < p.G;  // an odd G leaves the last pair's second half idle
  const int64_t nt = (p.M + EX_ROWS - 1) / EX_ROWS;
  const int64_t t0 = (int64_t)slice * nt / p.n_slices;
  const int64_t t1 = (int64_t)(slice + 1) * nt / p.n_slices;
  if (t0 >= t1) return;

  // W_g (512 x 128, [k][n]) transposed into LDS as [n][k], one group of the
  // pair at a time: in each round a wave reads 16 bytes (8 columns) of 64
  // consecutive k and writes them as 8 rows of 64 consecutive k; then the
  // group's four waves take their 32 columns as A operands (row n = 32 cw +
  // 16 cb + n16, K step c covers k = 32c + 8 g4 .. + 7)
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  bf16x8 wf[2][EX_DC / 32];
#pragma unroll
  for (int sel = 0; sel < 2; ++sel) {
    const int gs = 2 * gp + sel;
    if (gs >= p.G) break;  // uniform
    const uint16_t* wg = p.w + (size_t)gs * EX_DC * EX_N;
#pragma unroll 2
    for (int it = 0; it < (EX_DC / 64) * (EX_N / 8) / 8; ++it) {
      const int job = 8 * it + wave;  // (k block, column chunk)
      const int kb = job / (EX_N / 8), nc = job % (EX_N / 8);
      const int k = 64 * kb + lane;
      const u32x4 v = *(const u32x4*)(wg + (size_t)k * EX_N + 8 * nc);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint16_t x = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
        ((lds_u16*)(lds_p + (8 * nc + e) * EX_WPITCH))[k] = x;
      }
    }
    __syncthreads();
    if (half == sel) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int c = 0; c < EX_DC / 32; ++c)
          wf[cb][c] = *(const __attribute__((address_space(3))) bf16x8*)(
              lds_p + (32 * cw + 16 * cb + n16) * EX_WPITCH + 2 * (32 * c + 8 * g4));
    }
    __syncthreads();  // the staging area is rewritten, then becomes the tile buffers
  }

  // tile t's 72 KiB: copy i (wave w issues i = w, w + 8, ...) fills LDS
  // bytes 1024i .., 16-byte unit u = 64i + lane is chunk x of row r; rows
  // past the end repeat the last row (their products are never stored)
  auto issue_tile = [&](int64_t t, uint32_t dst) {
    const int64_t m0 = t * EX_ROWS;
    const int nv = (int)(p.M - m0 < EX_ROWS ? p.M - m0 : EX_ROWS);
    const char* pbase = uniform_ptr((const char*)p.a + m0 * EX_PITCH);
#pragma unroll
    for (int u = 0; u < EX_TILE / 1024 / 8; ++u) {
      const int i = wave + 8 * u;
      const int uu = 64 * i + lane;
      const int r = uu / 72, x = uu - 72 * r;
      dma16(dst + 1024 * i, pbase, min(r, nv - 1) * EX_PITCH + 16 * (x ^ (r & 7)));
    }
  };

  // B operand (latent rows as columns of A^T): row m = 16 kb + n16 of the
  // tile, chunk 4c + g4 at position (4c + g4) ^ (m & 7): with an XOR below 8
  // two base offsets (c even / odd) plus 128 (c >> 1) reach every step
  uint32_t a_off[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) a_off[q] = n16 * EX_PITCH + 16 * ((4 * q + g4) ^ (n16 & 7));

  // Outputs leave through LDS so that every store writes whole rows: once
  // every wave is done with tile t's products, each wave writes its 32
  // columns of the tile's 64 rows (bf16) into the tile's own buffer, group
  // half h at h * OUT_HALF, rows OUT_PITCH apart; then each wave stores 16
  // of its group's rows, four 256-byte rows per instruction.
  constexpr int OUT_PITCH = 2 * EX_N + 16;        // 128 bf16 + 16 bytes of bank skew
  constexpr int OUT_HALF = EX_ROWS * OUT_PITCH;
  static_assert(2 * OUT_HALF <= EX_TILE, "both groups' outputs fit a tile buffer");

  issue_tile(t0, lds0);
  wait_vm<0>();
  int cur = 0;
  for (int64_t t = t0; t < t1; ++t) {
    // every wave's copies of tile t have landed (each waited before the
    // previous tile's staging barrier) and every wave has stored its rows
    // of tile t - 1 out of the other buffer, which tile t + 1 now refills
    barrier();
    if (t + 1 < t1) issue_tile(t + 1, lds0 + (cur ^ 1) * EX_TILE);

    lds_char* const buf = lds_p + cur * EX_TILE;
    auto a_frag = [&](int st) -> bf16x8 {
      const int c = st / 4, kb = st % 4;
      return *(const __attribute__((address_space(3))) bf16x8*)(
          buf + a_off[c & 1] + kb * 16 * EX_PITCH + 128 * (c >> 1));
    };
    // C^T = W_g^T . A^T: step st = (c, kb) reads one latent fragment and
    // feeds both column blocks; consecutive MFMAs use different accumulators
    f32x4 acc[2][4];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) acc[cb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int NST = 4 * EX_DC / 32;
    bf16x8 af[EX_PF + 1];
#pragma unroll
    for (int st = 0; st < EX_PF; ++st) af[st] = a_frag(st);
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      if (st + EX_PF < NST) af[(st + EX_PF) % (EX_PF + 1)] = a_frag(st + EX_PF);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        acc[cb][st % 4] = mfma16(wf[cb][st / 4], af[st % (EX_PF + 1)], acc[cb][st % 4]);
      mem_fence_compiler();
    }
    const int64_t m0 = t * EX_ROWS;
    // K: the rope columns (chunks 64 .. 71 of the latent row, at positions
    // 64 + ((c - 64) ^ (r & 7))): thread j of the group's half takes row
    // j / 4, chunks 2 (j % 4) and 2 (j % 4) + 1, read before the staging
    // overwrites the tile
    u32x4 rope_v[2];
    const int j = tid & 255;
    if (p.rope) {
      const int r = j >> 2, c0 = 2 * (j & 3);
#pragma unroll
      for (int e = 0; e < 2; ++e)
        rope_v[e] = *(const __attribute__((address_space(3))) u32x4*)(
            buf + r * EX_PITCH + 16 * (64 + ((c0 + e) ^ (r & 7))));
    }
    // this wave's copies of tile t + 1 (issued before the products) and its
    // stores of tile t - 1 have completed, its LDS reads too; after the
    // barrier no wave reads tile t any more
    wait_vm<0>();
    wait_lgkm0();
    barrier();
    // lane l holds C[m = 64t + 16kb + l % 16][n = 32 cw + 16 cb + 4 (l / 16) + r]
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        u32x2 x;
        x[0] = pack_bf16x2(acc[cb][kb][0], acc[cb][kb][1]);
        x[1] = pack_bf16x2(acc[cb][kb][2], acc[cb][kb][3]);
        *(__attribute__((address_space(3))) u32x2*)(
            buf + half * OUT_HALF + (16 * kb + n16) * OUT_PITCH + 2 * (32 * cw + 16 * cb + 4 * g4)) = x;
      }
    wait_lgkm0();  // the staged rows are in LDS before any wave reads them
    barrier();
    if (live) {
      // rows 16 cw + 4 i + l / 16, 16 bytes l % 16 of each
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * cw + 4 * i + (lane >> 4);
        const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(
            buf + half * OUT_HALF + r * OUT_PITCH + 16 * (lane & 15));
        const int64_t m = m0 + r;
        if (m < p.M)
          *(u32x4*)(p.c + m * p.c_outer + (int64_t)g * p.c_batch + 8 * (lane & 15)) = v;
      }
      if (p.rope) {
        const int64_t m = m0 + (j >> 2);
        if (m < p.M) {
          uint16_t* dst = p.c + m * p.c_outer + (int64_t)g * p.c_batch + p.rope_c_off + 16 * (j & 3);
          *(u32x4*)dst = rope_v[0];
          *(u32x4*)(dst + 8) = rope_v[1];
        }
      }
    }
    cur ^= 1;
  }
}

}  // namespace

hipError_t launch_expand(const ExpandArgs& a, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  if (a.G < 1 || a.n_slices < 8 || a.n_slices % 8 != 0 ||
      (int64_t)((a.G + 1) / 2) * a.n_slices > 0x7fffffffLL)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(expand_kernel, dim3(((a.G + 1) / 2) * a.n_slices), dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace mla
