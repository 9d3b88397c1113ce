// Argument blocks and launchers shared by the kernels and the C interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Cache shapes of the decode kernel.
enum : int {
  KIND_MLA = 0,       // latent rows of 576 (V = the first 512 columns), one KV head
  KIND_GQA = 1,       // separate 128-wide K and V rows per KV head
  KIND_GQA_ROPE = 2,  // 192-wide K rows (128 + 64 rope) and 128-wide V rows per KV head
  KIND_MLA_FP8 = 3,   // latent rows of 576 E4M3 codes with one fp32 scale per token
};

struct DecodeArgs {
  const uint16_t* q;           // [B, T, H, D]
  const uint16_t* k;           // [P, 64, G, D]
  const uint16_t* v;           // [P, 64, G, DV]; null: V = K[..., :DV]
  const float* kscale;         // [P, 64] per-token scales of an FP8 cache, else null
  const int32_t* block_table;  // [B, bt_stride]
  const int32_t* seqlens;      // [B]
  const int32_t* meta;         // signature [HDR], worker records [W][REC], unit prefix [B + 1]
  const int32_t* slots;        // [B + 1] partial slots per sequence
  float* part_o;               // [slots][T*H][DV]
  float* part_lse;             // [slots][T*H]
  uint16_t* out;               // [B, T, H, DV]
  float* lse;                  // [B, T, H]
  int B, T, H, G, bt_stride;
  int M;                       // query rows per KV head: T * H / G
  int nrb;                     // row blocks per KV head
  int W;                       // workers
  float scale_log2;            // softmax scale * log2(e)
  int causal;
};

struct CombineArgs {
  const int32_t* meta;         // the plan's metadata (its signature is checked), or null
  int W, G;                    // workers and KV heads of the decode call (with meta)
  const float* part_o;         // [slots][R][DV]
  const float* part_lse;       // [slots][R]
  const int32_t* slots;        // [B + 1]
  uint16_t* out;               // [B][R][DV]
  float* lse;                  // [B][R]
  int B, R, DV;
  // Merge in one pass (level 0), or in two launches for sequences with many
  // partials: level 1 merges chunk z < Z of ceil(n / Z) consecutive partials
  // into the chunk's first slot of chunk_o / chunk_lse (the same buffers as
  // part_o / part_lse), level 2 merges the chunks' results into out / lse.
  int level, Z;
  int wide;  // one pass with four partial rows in flight instead of two
  float* chunk_o;
  float* chunk_lse;
};

struct AppendArgs {
  const char* src0;            // [B, T] rows of row_bytes (MLA rows, or GQA K)
  const char* src1;            // GQA V rows, or null
  char* dst0;                  // cache [P, 64] rows of row_bytes
  char* dst1;                  // GQA V cache, or null
  const int32_t* block_table;  // [B, bt_stride]
  const int32_t* seqlens;      // [B], counting the T new tokens
  size_t row_bytes;            // a multiple of 16
  int B, T, bt_stride, num_pages;
};

// C = A . B on bf16 MFMA with fp32 accumulation, rounded to bf16, for a
// batch of problems (blockIdx.y). Row m of A (and of C) in problem z starts
// at  base + z * batch + (m / inner) * outer + (m % inner) * inner_stride
// (elements); rows hold K (A) or N (C) contiguous elements. B of problem z
// starts at b + z * b_batch and is [N][ldb] with K contiguous (b_kn = 0) or
// [K][ldb] with N contiguous (b_kn = 1). N % 128 == 0, K % 64 == 0. With
// rope set, each C row also gets 64 elements copied from its A row:
// C[row][rope_c_off + e] = A[row][rope_a_off + e], e < 64.
struct GemmArgs {
  const uint16_t* a;
  const uint16_t* b;
  uint16_t* c;
  int64_t a_outer, a_inner, a_batch;
  int64_t b_batch;
  int64_t c_outer, c_inner, c_batch;
  int ldb, inner, M, N, K, batches, b_kn;
  int rope, rope_a_off, rope_c_off;
};

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);

// GQLA cache expansion: C[m, g, 0:128] = A[m, 0:512] W_g (A rows of 576
// bf16, W [G][512][128]); with rope, also C[m, g, rope_c_off + j] =
// A[m, 512 + j] for j < 64. Grid G * n_slices (n_slices a multiple of 8).
struct ExpandArgs {
  const uint16_t* a;      // [M, 576]
  const uint16_t* w;      // [G, 512, 128]
  uint16_t* c;            // row m, group g at c + m * c_outer + g * c_batch
  int64_t M, c_outer;
  int G, c_batch, rope, rope_c_off, n_slices;
};
hipError_t launch_expand(const ExpandArgs& a, hipStream_t st);

// FP8 quantisation of 576-wide bf16 latent rows: row r of src (r < B * T)
// goes to row r of dst (block_table null), or, as an append, to the slot of
// new token t = r % T of sequence b = r / T (same rule as AppendArgs).
struct QuantArgs {
  const uint16_t* src;         // [B * T, 576] bf16
  uint8_t* codes;              // [rows or P * 64, 576] E4M3
  float* scales;               // [rows or P * 64]
  const int32_t* block_table;  // [B, bt_stride] or null
  const int32_t* seqlens;      // [B] (append only)
  int B, T, bt_stride, num_pages;
};

hipError_t launch_quantize_fp8(const QuantArgs& a, hipStream_t st);

// Paged KV append: one wave per new token.
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t st);

// The latent decode at 128 query rows per workgroup (32x32x16 MFMA, four
// waves of 32 rows): grid = workers * row blocks of 128.
hipError_t launch_decode128_kernel(const DecodeArgs& a, int grid, hipStream_t st);
// One decode launch: grid = workers * row blocks, 64 * nw threads.
hipError_t launch_decode_kernel(const DecodeArgs& a, int nw, int kind, int grid, hipStream_t st);
// Split-KV merge of the partial results of split sequences (one level, or
// the two launches of levels 1 and 2 when a.Z > 1).
hipError_t launch_combine_kernel(const CombineArgs& a, hipStream_t st);
// Device-side precondition check of the decode calls (one workgroup).
hipError_t launch_check_fp8_scales(const float* scales, int64_t n, int32_t* status,
                                   hipStream_t st);
hipError_t launch_check_pages(const int32_t* block_table, const int32_t* seqlens, int B,
                              int num_pages, int max_pages, int32_t* status, hipStream_t st);
// Schedule: signature, worker records and unit prefix into meta, slot
// prefix into slots.
hipError_t launch_plan_kernel(const int32_t* seqlens, int B, int W, int rows, int G, int DV,
                              int fix, int32_t* meta, int32_t* slots, hipStream_t st);

}  // namespace mla
