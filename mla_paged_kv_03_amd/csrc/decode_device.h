// Device helpers shared by the decode kernels: workgroup numbering, the
// LDS page layouts, HBM -> LDS copies, wait counts, barriers and wave
// reductions.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace mla {

// Map a workgroup id to (worker, row block). Workgroups are dispatched to
// the 8 XCDs round-robin, so the row blocks of one worker (which read the
// same pages) get ids congruent mod 8 and share an XCD's L2.
__device__ __forceinline__ void decode_block_id(int bid, int W, int RB, int& w, int& rb) {
  if ((W & 7) == 0) {
    const int group = bid / (8 * RB);
    const int rem = bid - group * 8 * RB;
    rb = rem >> 3;
    w = group * 8 + (rem & 7);
  } else {
    w = bid / RB;
    rb = bid - w * RB;
  }
}

// Map a workgroup id to (worker, row block) with each XCD holding a
// contiguous run of W / 8 workers, all row blocks of each: besides the row
// blocks of a worker, the neighbouring workers that share the pieces of one
// split sequence (and so its queries) then share an XCD's L2.
__device__ __forceinline__ void decode_block_id_xcd(int bid, int W, int RB, int& w, int& rb) {
  if ((W & 7) == 0) {
    const int x = bid & 7, k = bid >> 3;
    const int kw = k / RB;
    rb = k - kw * RB;
    w = x * (W >> 3) + kw;
  } else {
    w = bid / RB;
    rb = bid - w * RB;
  }
}

// Waves per decode workgroup: four compute waves, plus four copy waves for
// the latent cache at 64 query rows per workgroup (bf16, or FP8 pages that
// the copy waves dequantise to bf16), where every page is copied once per
// row block and the copies cost the compute waves as much time as the
// products when they issue them themselves.
constexpr int decode_waves(int R, int KIND) {
  return ((KIND == KIND_MLA || KIND == KIND_MLA_FP8) && R == 4) ? 8 : 4;
}

// LDS page layouts (bytes). Row k of a page keeps its 16-byte chunk c at
// k * PITCH + 16 * (c ^ xor(k)). Measured on gfx950 (whose LDS serves 256
// bytes per clock), these choices let the K-operand reads (16 rows x 16 bytes
// per 16-lane group) run at the full LDS rate and the transposed V reads (4
// rows x 32 bytes per group) at their best rate; a 3-bit XOR over 1 KiB rows
// ran both at about half of that. An XOR below 8 keeps a chunk inside its
// aligned group of 8 chunks (K_XOR8 / V_XOR8), so one lane offset serves
// every group of a row; a 4-bit XOR needs one offset per chunk position.
template <int KIND>
struct Layout;

// Latent cache: a page is copied as it lies in HBM, 64 rows of 1152 bytes:
// columns 0..511 (latent, which is also V) in chunks 0..63, the rope columns
// 512..575 in chunks 64..71.
template <>
struct Layout<KIND_MLA> {
  static constexpr int D = 576, DV = 512;
  static constexpr int K_PITCH = 1152, V_PITCH = 1152;
  static constexpr int TILE = 64 * K_PITCH;  // one page
  static constexpr int V_BASE = 0;
  static constexpr int DMA_PER_TILE = 72;  // 1 KiB per instruction
  static constexpr int NBUF = 2;           // page buffers (2 x 72 KiB)
  static constexpr bool K_XOR8 = true, V_XOR8 = true;
  static constexpr bool FP8 = false;
  static __device__ __forceinline__ int k_xor(int k) { return k & 7; }
  static __device__ __forceinline__ int v_xor(int k) { return k & 7; }
};

// GQA: separate 128-wide K and V rows (256 bytes, 16 chunks) of one KV head;
// the XOR 2 (k & 7) stays inside the row.
template <>
struct Layout<KIND_GQA> {
  static constexpr int D = 128, DV = 128;
  static constexpr int K_PITCH = 256, V_PITCH = 256;
  static constexpr int TILE = 2 * 64 * 256;
  static constexpr int V_BASE = 64 * 256;
  static constexpr int DMA_PER_TILE = 32;
  static constexpr int NBUF = 2;
  static constexpr bool K_XOR8 = false, V_XOR8 = false;
  static constexpr bool FP8 = false;
  static __device__ __forceinline__ int k_xor(int k) { return (k & 7) << 1; }
  static __device__ __forceinline__ int v_xor(int k) { return (k & 7) << 1; }
};

// GQA with decoupled rope: 192-wide K rows (128 group columns + the 64 rope
// columns, 384 bytes = 24 chunks) and 128-wide V rows. A 384-byte pitch puts
// rows 16 bytes x 8 apart modulo the 256 LDS bytes, as the 1152-byte latent
// rows are, so K takes the latent layout's XOR and V the GQA one. Two page
// buffers take 80 KiB: two workgroups share a CU.
template <>
struct Layout<KIND_GQA_ROPE> {
  static constexpr int D = 192, DV = 128;
  static constexpr int K_PITCH = 384, V_PITCH = 256;
  static constexpr int TILE = 64 * 384 + 64 * 256;
  static constexpr int V_BASE = 64 * 384;
  static constexpr int DMA_PER_TILE = 40;
  static constexpr int NBUF = 2;
  static constexpr bool K_XOR8 = true, V_XOR8 = false;
  static constexpr bool FP8 = false;
  static __device__ __forceinline__ int k_xor(int k) { return k & 7; }
  static __device__ __forceinline__ int v_xor(int k) { return (k & 7) << 1; }
};

// FP8 latent cache: 64 rows of 576 E4M3 codes (36 chunks of 16 bytes), then
// the page's 64 fp32 token scales. Chunk c of row k sits at chunk
// c ^ fp8_xor(k), an XOR below 4 (inside aligned groups of 4 chunks):
// bits 3-4 of the row spread the 16 rows of a score read (8 bytes each, rows
// 576 bytes = 16 banks apart, so rows k and k + 4 would collide) over the
// banks, and bit 2 separates rows k and k + 4 of a transposed V read.
template <>
struct Layout<KIND_MLA_FP8> {
  static constexpr int D = 576, DV = 512;
  static constexpr int K_PITCH = 576, V_PITCH = 576;
  static constexpr int SCALE_OFF = 64 * 576;
  static constexpr int TILE = SCALE_OFF + 256;
  static constexpr int V_BASE = 0;
  static constexpr int DMA_PER_TILE = 36 + 4;  // codes, plus one scale copy per wave
  // half-size pages: four buffers (145 KiB) keep three pages in flight
  static constexpr int NBUF = 4;
  static constexpr bool K_XOR8 = true, V_XOR8 = true;
  static constexpr bool FP8 = true;
  static __device__ __forceinline__ int k_xor(int k) { return ((k >> 3) & 3) ^ (((k >> 2) & 1) << 1); }
  static __device__ __forceinline__ int v_xor(int k) { return k_xor(k); }
};

// Issue one 1 KiB HBM -> LDS copy: lane l's 16 bytes at sbase + voff land at
// LDS byte lds + 16 * l. Issued from inline asm so that the compiler does not
// add its own conservative wait on the asynchronous LDS write; the kernel
// waits with explicit vmcnt counts.
// The compiler does not insert hazard wait states inside inline asm, so the
// block carries its own: a VALU write of an SGPR (readfirstlane of the base)
// needs 5 wait states before a vector memory instruction reads that SGPR, and
// an SALU write of M0 needs 1 before an LDS DMA reads M0. The copy is marked
// non-temporal (nt): each cache byte is read once per workgroup, and the hint
// lifted the HBM-bound shapes by about 10 % on the device.
__device__ __forceinline__ void dma16(uint32_t lds, const void* sbase, uint32_t voff) {
  asm volatile("s_nop 4\n\ts_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :
               : "s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// One 256-byte HBM -> LDS copy: lane l's 4 bytes at sbase + voff land at LDS
// byte lds + 4 * l (same wait states as dma16).
__device__ __forceinline__ void dma4(uint32_t lds, const void* sbase, uint32_t voff) {
  asm volatile("s_nop 4\n\ts_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2 nt"
               :
               : "s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// Two E4M3 codes (bytes 0-1, or 2-3 with HI) of w as two bf16 in one word,
// exactly (every E4M3 value is a bf16 value). Only whole words are used:
// the pair is never split into elements.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// The same two codes times s, rounded to bf16 (to nearest even) by the
// conversion itself; with a power-of-two s the product is exact inside the
// bf16 range.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16x2_scaled(uint32_t w, float s) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, s, HI));
}
__device__ __forceinline__ bf16x8 fp8x8_bf16x8(uint32_t w0, uint32_t w1) {
  const u32x4 u = {fp8x2_bf16x2<false>(w0), fp8x2_bf16x2<true>(w0), fp8x2_bf16x2<false>(w1),
                   fp8x2_bf16x2<true>(w1)};
  return __builtin_bit_cast(bf16x8, u);
}

// LDS operand reads are issued this many MFMA steps ahead of their use.
#ifndef MLA_LDS_PREFETCH
#define MLA_LDS_PREFETCH 6
#endif
constexpr int PF = MLA_LDS_PREFETCH;

// Softmax weights may exceed 1 by up to 2^RESCALE_SLACK before O is rescaled.
constexpr float RESCALE_SLACK = 8.f;
// With a fixed reference, weights up to 2^REF_LIMIT are accepted: sums of up
// to 2^60 such terms times |V| stay far inside the fp32 range.
constexpr float REF_LIMIT = 64.f;

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Keeps the compiler from moving memory operations across this point (it
// bounds how far LDS reads are hoisted ahead of the MFMAs that use them).
__device__ __forceinline__ void mem_fence_compiler() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uintptr_t u = (uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const T*)(((uintptr_t)hi << 32) | lo);
}

// Scalar load of one int32 from a wave-uniform address. The wait sits in the
// same asm statement, so the result is ready when the statement ends; it is
// a scalar-cache load and does not touch vmcnt, which counts page copies.
// The block opens with one wait state after a possible VALU write of the
// address registers (a v_readfirstlane or v_readlane just before it).
__device__ __forceinline__ int sload(const int32_t* p) {
  int v;
  asm volatile("s_nop 0\n\ts_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p)
               : "memory");
  return v;
}

__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Block-wide OR of a per-lane flag, through the first words of the page
// buffers. Called only where those are idle: every copy has landed and every
// wave has passed the page loop's last barrier. (The runtime's own
// __syncthreads_or keeps 256 bytes of LDS of its own, which would leave the
// 80 KiB page buffers of the rope layout one workgroup per CU.)
template <int NW>
__device__ __forceinline__ bool block_or(bool x, lds_char* lds_p, int wave) {
  typedef __attribute__((address_space(3))) int lds_int;
  lds_int* f = (lds_int*)lds_p;
  const int any = __any(x) ? 1 : 0;
  if ((threadIdx.x & 63) == 0) f[wave] = any;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) r |= f[w];
  __syncthreads();  // the words are page data again afterwards
  return r != 0;
}

// Reductions over the four 16-lane groups (lanes l, l ^ 16, l ^ 32,
// l ^ 48) with gfx950's lane swaps, which stay in the VALU: swapping the odd
// 16-lane rows of one copy of x with the even rows of another leaves
// {x[l], x[l ^ 16]} in the two results of lane l (the 32-lane swap likewise
// {x[l], x[l ^ 32]}), and the pair's max or sum is the same in both lanes.
__device__ __forceinline__ float max4groups(float x) {
  uint32_t u = __float_as_uint(x);
  auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  u = __float_as_uint(x);
  p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum4groups(float x) {
  uint32_t u = __float_as_uint(x);
  auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  u = __float_as_uint(x);
  p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

}  // namespace mla
