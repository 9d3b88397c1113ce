// GQLA's cache expansion, the GQA path's K and V pages from the latent
// rows (GQLA review, "2. Motivation & Problem Statement": the up-projections
// are indexed by KV group): for every latent row m and group g,
//     C[m, g, 0:128] = A[m, 0:512] . W_g            (W_g: 512 x 128)
// and, for K, C[m, g, 128:192] = A[m, 512:576] (the shared rope columns).
//
// The product has the shape of the decode kernel's score product with the
// roles renamed: latent rows for keys, the 128 weight columns of a group for
// query rows, the 512 latent columns for the head dimension. So the kernel
// is laid out like the decode kernel: a workgroup keeps one group's weights
// in registers (each wave 32 columns, 128 VGPRs) and streams 64-row tiles of
// latent rows HBM -> LDS in the decode page layout (rows of 1152 bytes, 16-
// byte chunk c of row r at c ^ (r & 7)), two buffers, the next tile in
// flight while one is multiplied. As in the decode kernel, four copy waves
// issue the tile copies and four compute waves run the MFMAs, meeting at
// one barrier per tile. Every latent tile crosses into a CU once per group;
// the weights are read once per workgroup.
//
// Work: the groups' workgroups of one slice of rows get ids congruent mod 8,
// so they run on one XCD (round-robin dispatch) and read the slice's tiles
// through the same L2.
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
  const bool copier = wave >= 4;  // waves 4 .. 7 copy tiles, waves 0 .. 3 compute

  // workgroup id -> (group, slice of rows); the grid is G * n_slices and
  // n_slices is a multiple of 8
  const int xcd = blockIdx.x & 7, t8 = blockIdx.x >> 3;
  const int g = t8 % p.G;
  const int slice = (t8 / p.G) * 8 + xcd;
  const int64_t nt = (p.M + EX_ROWS - 1) / EX_ROWS;
  const int64_t t0 = (int64_t)slice * nt / p.n_slices;
  const int64_t t1 = (int64_t)(slice + 1) * nt / p.n_slices;
  if (t0 >= t1) return;

  // W_g (512 x 128, [k][n]) transposed into LDS as [n][k]: in each round a
  // wave reads 16 bytes (8 columns) of 64 consecutive k and writes them as
  // 8 rows of 64 consecutive k
  const uint16_t* wg = p.w + (size_t)g * EX_DC * EX_N;
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
#pragma unroll 4
  for (int it = 0; it < (EX_DC / 64) * (EX_N / 8) / 4 && !copier; ++it) {
    const int job = 4 * it + wave;  // (k block, column chunk)
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
  // this wave's 32 columns as A operands: row n = 32 wave + 16 cb + n16,
  // K step c covers k = 32c + 8 g4 .. + 7
  bf16x8 wf[2][EX_DC / 32];
  if (!copier) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int c = 0; c < EX_DC / 32; ++c)
        wf[cb][c] = *(const __attribute__((address_space(3))) bf16x8*)(
            lds_p + (32 * wave + 16 * cb + n16) * EX_WPITCH + 2 * (32 * c + 8 * g4));
  }
  __syncthreads();  // the staging area becomes the tile buffers

  // tile t's 72 KiB: copy i fills LDS bytes 1024i .., 16-byte unit u =
  // 64i + lane is chunk x of row r; rows past the end repeat the last row
  // (its products are never stored)
  auto issue_tile = [&](int64_t t, uint32_t dst) {
    const int64_t m0 = t * EX_ROWS;
    const int nv = (int)(p.M - m0 < EX_ROWS ? p.M - m0 : EX_ROWS);
    const char* pbase = uniform_ptr((const char*)p.a + m0 * EX_PITCH);
#pragma unroll
    for (int u = 0; u < EX_TILE / 1024 / 4; ++u) {
      const int i = (wave - 4) + 4 * u;
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

  if (copier) {
    // At the barrier opening tile t, each copy wave has waited for its own
    // copies of tile t and every compute wave has finished tile t - 1, whose
    // buffer then takes tile t + 1.
    issue_tile(t0, lds0);
    int cur = 0;
    for (int64_t t = t0; t < t1; ++t) {
      wait_vm<0>();
      barrier();
      if (t + 1 < t1) issue_tile(t + 1, lds0 + (cur ^ 1) * EX_TILE);
      cur ^= 1;
    }
    return;
  }
  int cur = 0;
  for (int64_t t = t0; t < t1; ++t) {
    barrier();

    const lds_char* buf = lds_p + cur * EX_TILE;
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

    // lane l holds C[m = 64t + 16kb + l % 16][n = 32 wave + 16 cb + 4 (l / 16) + r]
    const int64_t m0 = t * EX_ROWS;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int64_t m = m0 + 16 * kb + n16;
      if (m >= p.M) continue;
      uint16_t* crow = p.c + m * p.c_outer + (int64_t)g * p.c_batch + 32 * wave + 4 * g4;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        u32x2 x;
        x[0] = pack_bf16x2(acc[cb][kb][0], acc[cb][kb][1]);
        x[1] = pack_bf16x2(acc[cb][kb][2], acc[cb][kb][3]);
        *(u32x2*)(crow + 16 * cb) = x;
      }
    }
    // K: the rope columns of the tile's rows (chunks 64 .. 71 of the latent
    // row, at positions 64 + ((c - 64) ^ (r & 7))) to columns 128 .. 191
    if (p.rope) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int idx = tid + 256 * e;
        const int r = idx >> 3, ch = idx & 7;
        const int64_t m = m0 + r;
        if (m >= p.M) continue;
        const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(
            buf + r * EX_PITCH + 16 * (64 + (ch ^ (r & 7))));
        *(u32x4*)(p.c + m * p.c_outer + (int64_t)g * p.c_batch + p.rope_c_off + 8 * ch) = v;
      }
    }
    cur ^= 1;
  }
}

}  // namespace

hipError_t launch_expand(const ExpandArgs& a, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  if (a.G < 1 || a.n_slices < 8 || a.n_slices % 8 != 0 ||
      (int64_t)a.G * a.n_slices > 0x7fffffffLL)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(expand_kernel, dim3(a.G * a.n_slices), dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace mla
