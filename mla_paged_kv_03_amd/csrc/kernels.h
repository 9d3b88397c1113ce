// Argument blocks and launchers shared by the kernels and the C interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct DecodeArgs {
  const uint16_t* q;           // [B, T, H, D]
  const uint16_t* k;           // [P, 64, G, D]
  const uint16_t* v;           // [P, 64, G, DV]; null: V = K[..., :DV]
  const int32_t* block_table;  // [B, bt_stride]
  const int32_t* seqlens;      // [B]
  const int32_t* meta;         // worker records [W][REC], then unit prefix [B + 1]
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
  const float* part_o;         // [slots][R][DV]
  const float* part_lse;       // [slots][R]
  const int32_t* slots;        // [B + 1]
  uint16_t* out;               // [B][R][DV]
  float* lse;                  // [B][R]
  int B, R, DV;
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

// Paged KV append: one wave per new token.
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t st);

// One decode launch: grid = workers * row blocks, 64 * nw threads.
hipError_t launch_decode_kernel(const DecodeArgs& a, int nw, bool gqa, int grid, hipStream_t st);
// Split-KV merge of the partial results of split sequences.
hipError_t launch_combine_kernel(const CombineArgs& a, hipStream_t st);
// Schedule: worker records and unit prefix into meta, slot prefix into slots.
hipError_t launch_plan_kernel(const int32_t* seqlens, int B, int W, int32_t* meta,
                              int32_t* slots, hipStream_t st);

}  // namespace mla
