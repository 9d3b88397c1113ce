/*
 * Paged attention decode on MI355X (gfx950): C interface.
 *
 * What is computed. For every sequence b, query token t and query head h:
 *     out[b,t,h,:] = sum_j softmax_j(scale * q[b,t,h,:] . K_b[j,g,:]) V_b[j,g,:]
 *     lse[b,t,h]   = ln sum_j exp(scale * q[b,t,h,:] . K_b[j,g,:])
 * the attention of FlashAttention (KO), section "표준 Attention의 문제점",
 * computed exactly (section "온라인 Softmax 계산": running max and running
 * exp-sum) in one fused pass per 64-token page, so the score matrix never
 * reaches HBM (sections "타일링 및 블록 처리" and "단일 CUDA 커널로의 연산 융합").
 * j runs over the keys query token t may see: 0 <= j < L_b, and with
 * causal != 0, j <= L_b - s_q + t (the s_q new tokens are the last s_q of
 * the L_b cached ones). A row that sees no key gets out = 0, lse = -inf.
 *
 * The cache is paged: token j of sequence b lives in physical page
 * block_table[b, j / 64], slot j % 64 (PagedAttention, cited in the same
 * article's "참고 문헌"; 64-token pages per the FlashMLA blog, "기술 기반").
 * Two shapes (GQLA review, "1. Key Terms & Definitions"):
 *   - mla_decode: MQA-absorb path. One latent KV head; every query head
 *     attends the same 576-wide row (512 latent + 64 rope) and V is its
 *     first 512 columns.
 *   - gqa_decode: GQA path. h_kv KV heads with separate 128-wide K and V;
 *     query head h uses KV head h / (h_q / h_kv).
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless marked (host). The caller owns
 *     every buffer; the library keeps only a per-device cache of the
 *     compute-unit count.
 *   - bf16 tensors are contiguous, row-major in the shapes given, 16-byte
 *     aligned. int32 tensors are contiguous.
 *   - Work is enqueued on `stream` (0 = the null stream). No call blocks,
 *     allocates device memory or copies device data to the host.
 *   - Return value: MLA_OK (0) or a negative MLA_ERR_* code. Every argument
 *     check happens before anything is enqueued; on error nothing is.
 *   - Device-resident data cannot be checked from the host; these are
 *     preconditions: 0 <= cache_seqlens[b] <= 64 * max_pages_per_seq, and
 *     0 <= block_table[b, j] < num_pages for j < ceil(cache_seqlens[b] / 64).
 *     Block-table entries past that (pads, e.g. -1) are never read, and
 *     neither are page slots at or past cache_seqlens[b].
 *   - Split-KV: one launch spreads the pages of all sequences evenly over a
 *     fixed number of workgroups (mla_decode_plan). A sequence whose pages
 *     land on several workgroups is finished by an internal log-sum-exp
 *     merge (attn_combine's kernel) inside the same call.
 */
#ifndef MLA_DECODE_H_
#define MLA_DECODE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MLA_OK = 0,
  MLA_ERR_NULL_ARG = -1,            /* a required pointer is NULL */
  MLA_ERR_BAD_SHAPE = -2,           /* negative size, h_q % h_kv != 0, ... */
  MLA_ERR_UNSUPPORTED = -3,         /* head dims or row counts not built */
  MLA_ERR_WORKSPACE_TOO_SMALL = -4, /* workspace_bytes below the plan's */
  MLA_ERR_HIP = -5,                 /* a HIP runtime call or launch failed */
  MLA_ERR_SCRATCH_LIMIT = -6        /* mla_decode_noalloc: needs more than its static scratch */
};

/* Host-side description of a decode plan, filled by mla_decode_plan. */
typedef struct {
  int32_t num_workers;      /* workgroups that share the pages of the batch */
  int32_t row_blocks;       /* workgroups per worker (query-row blocks x KV heads) */
  int32_t max_split_slots;  /* upper bound of partial results (2 * (workers - 1)) */
  int32_t reserved;
  size_t metadata_bytes;    /* size of sched_metadata (int32) */
  size_t num_splits_bytes;  /* size of num_splits: (batch + 1) int32 */
  size_t workspace_bytes;   /* fp32 partials for split sequences */
} mla_plan_info;

/* Plan the split-KV schedule of one decode step (FlashAttention (KO),
 * section "FlashAttention-2 (2023)": better work partitioning across the
 * GPU; variable lengths per the FlashMLA blog, "기술 기반").
 *
 * The concatenated work of the batch, sum_b (ceil(L_b / 64) + 2) units,
 * is cut into num_workers nearly equal contiguous ranges; a sequence that
 * straddles a cut is split, and its partial results are merged later.
 *
 *   cache_seqlens  int32 [batch], device.
 *   batch, s_q, h_q, h_kv, head_dim_v: shape of the step (h_kv = 1 and
 *                  head_dim_v = 512 for mla_decode; h_kv > 1 and
 *                  head_dim_v = 128 for gqa_decode).
 *   sched_metadata int32 buffer of info->metadata_bytes (out).
 *   num_splits     int32 [batch + 1] (out): num_splits[b + 1] - num_splits[b]
 *                  is the number of partial results of sequence b (0 when
 *                  it is not split); num_splits[b] is its first slot.
 *   info           (host, out) sizes; required.
 *
 * With sched_metadata and num_splits both NULL only *info is filled and
 * nothing is enqueued, so callers can size buffers first. The sizes depend
 * only on the shape arguments and the current device. The plan may be
 * reused by every layer of the step (same cache_seqlens and shape).
 *
 * sched_metadata opens with 8 int32 words that record the geometry the plan
 * was made for: a fixed tag 0x4D4C4150, the worker count, batch, s_q * h_q,
 * h_kv and head_dim_v, then the plan's overhead units per piece of a
 * sequence and the batch's total cost in units. The decode kernels and their
 * internal merge compare this signature with their own call before they
 * read any worker record or slot; on a mismatch (a plan made for another
 * batch, s_q * h_q, h_kv, value width or device) they return at once and
 * leave out and lse unwritten. The call itself still returns MLA_OK: the
 * check runs on the device. A plan made for the same shape but other
 * cache_seqlens (a stale plan) gives undefined results, but every page range
 * is clamped to the current lengths, so no block-table entry or page slot
 * outside what the current lengths reach is read.
 */
int mla_decode_plan(const int32_t* cache_seqlens, int32_t batch, int32_t s_q,
                    int32_t h_q, int32_t h_kv, int32_t head_dim_v,
                    int32_t* sched_metadata, int32_t* num_splits,
                    mla_plan_info* info, hipStream_t stream);

/* The plan for mla_decode_fp8 (h_kv = 1, head_dim_v = 512), otherwise as
 * mla_decode_plan. The FP8 decode holds 64 query rows per workgroup at any
 * row count. From 128 rows per KV head on (s_q * h_q >= 128) its plan
 * therefore has one worker per CU and row block of 64 (a worker's pages are
 * taken by one workgroup per row block), where mla_decode_plan plans one
 * worker of 128 rows per CU for the bf16 decode; below 128 rows the two
 * plans are the same. From 128 rows on, a plan from the other call fails
 * the decode's signature check (out and lse are left unwritten, as for any
 * mismatched plan). */
int mla_decode_plan_fp8(const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t h_q,
                        int32_t* sched_metadata, int32_t* num_splits, mla_plan_info* info,
                        hipStream_t stream);

/* MLA decode, MQA-absorb path (GQLA review, "1. Key Terms & Definitions").
 *
 *   q              bf16 [batch, s_q, h_q, 576]
 *   kv_cache       bf16 [num_pages, 64, 1, 576]; V = columns 0..511
 *   block_table    int32 [batch, max_pages_per_seq]
 *   cache_seqlens  int32 [batch]
 *   softmax_scale  multiplies q.k before the softmax (1/sqrt(192) for
 *                  DeepSeek-V3 shapes)
 *   causal         0 or 1, see the top of this file
 *   sched_metadata, num_splits: from mla_decode_plan with the same
 *                  cache_seqlens, batch, s_q, h_q, h_kv = 1, head_dim_v = 512
 *   workspace      device scratch of at least info.workspace_bytes (may be
 *                  NULL when that is 0); contents on entry do not matter
 *   out            bf16 [batch, s_q, h_q, 512] (out)
 *   lse            fp32 [batch, s_q, h_q] (out), natural log
 * Supported: 1 <= s_q * h_q <= 2^20; rows are cut into blocks of 64.
 */
int mla_decode(const void* q, const void* kv_cache, const int32_t* block_table,
               const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t h_q,
               int32_t num_pages, int32_t max_pages_per_seq, float softmax_scale,
               int32_t causal, const int32_t* sched_metadata, const int32_t* num_splits,
               void* workspace, size_t workspace_bytes, void* out, float* lse,
               hipStream_t stream);

/* mla_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same plan, decode and merge kernels, with the plan's metadata, its
 * slot prefix and the split partials in a static device array of the
 * library (137 MiB per GPU, allocated when the library's code is loaded on
 * that GPU and held until the process ends) instead of caller buffers.
 *
 * Arguments as for mla_decode, without the plan and workspace. The call
 * enqueues the plan kernel, the decode and (when a sequence is split) the
 * merge on `stream`, and calls no allocating routine. Limits: 512 KiB of
 * plan metadata and slot prefix each (batch up to about 128k sequences)
 * and 136 MiB of partials, which every s_q * h_q fits on a 256-CU GPU;
 * larger calls return MLA_ERR_SCRATCH_LIMIT before anything is enqueued.
 * Every call on one GPU uses that GPU's one array, and each call leaves
 * its contents behind: two calls on one GPU whose work overlaps in time
 * (on different streams, or from different host threads) race and give
 * undefined results. Calls in order on one stream are safe.
 */
int mla_decode_noalloc(const void* q, const void* kv_cache, const int32_t* block_table,
                       const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t h_q,
                       int32_t num_pages, int32_t max_pages_per_seq, float softmax_scale,
                       int32_t causal, void* out, float* lse, hipStream_t stream);

/* GQA decode with a per-group expanded cache (GQLA review, "1. Key Terms &
 * Definitions", GQA path).
 *
 *   q              bf16 [batch, s_q, h_q, 128]
 *   k_cache        bf16 [num_pages, 64, h_kv, 128]
 *   v_cache        bf16 [num_pages, 64, h_kv, 128]
 *   out            bf16 [batch, s_q, h_q, 128] (out); lse fp32 [batch, s_q, h_q]
 *   The plan must come from mla_decode_plan with the same h_kv and
 *   head_dim_v = 128. Other arguments as for mla_decode.
 * Supported: h_q % h_kv == 0, any s_q * h_q / h_kv >= 1.
 */
int gqa_decode(const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_table, const int32_t* cache_seqlens, int32_t batch,
               int32_t s_q, int32_t h_q, int32_t h_kv, int32_t num_pages,
               int32_t max_pages_per_seq, float softmax_scale, int32_t causal,
               const int32_t* sched_metadata, const int32_t* num_splits, void* workspace,
               size_t workspace_bytes, void* out, float* lse, hipStream_t stream);

/* Merge partial attention results computed over disjoint key subsets of
 * the same rows (follows from the online-softmax statistics of
 * FlashAttention (KO), "온라인 Softmax 계산"): for every row with n >= 1
 * partials, lse = m + ln sum_i exp(lse_i - m) with m = max_i lse_i, and
 * out = sum_i exp(lse_i - lse) o_i; partials with lse_i = -inf add nothing,
 * and a row whose partials are all -inf gets out = 0, lse = -inf.
 *
 *   o_partial    fp32 [num_slots, rows_per_batch, dv], each partial already
 *                normalised over its own keys
 *   lse_partial  fp32 [num_slots, rows_per_batch], natural log
 *   num_splits   int32 [batch + 1], device: sequence b owns slots
 *                num_splits[b] .. num_splits[b + 1] - 1; a sequence with no
 *                slot is left untouched in out and lse
 *   out          bf16 [batch, rows_per_batch, dv] (out)
 *   lse          fp32 [batch, rows_per_batch] (out)
 * dv must be a multiple of 8, at most 1024.
 */
int attn_combine(const float* o_partial, const float* lse_partial, const int32_t* num_splits,
                 int32_t batch, int32_t rows_per_batch, int32_t dv, void* out, float* lse,
                 hipStream_t stream);

/* Paged KV append: the step before decode that puts the s_q new tokens'
 * cache rows into the paged cache (the KV cache kept in 64-token pages of
 * the FlashMLA blog, "기술 기반"; KV Cache and PagedAttention among the
 * related techniques of the Flash Attention wiki note, "지식 연결 (Graph)").
 * cache_seqlens counts the new tokens, as in mla_decode: new token t of
 * sequence b is position p = cache_seqlens[b] - s_q + t and goes to page
 * block_table[b, p / 64], slot p % 64. A token with p < 0 (a sequence
 * shorter than s_q) is not written; a block-table entry outside
 * [0, num_pages) is skipped rather than written through. Only the new
 * tokens' slots change; the copy is exact (bytes).
 *
 *   new_kv        bf16 [batch, s_q, 576] (in)
 *   kv_cache      bf16 [num_pages, 64, 1, 576] (in/out)
 *   block_table, cache_seqlens, num_pages, max_pages_per_seq: as for
 *                 mla_decode (device, int32)
 * Errors: MLA_ERR_BAD_SHAPE for negative sizes, s_q < 1 or unaligned
 * tensors; MLA_ERR_NULL_ARG for a NULL pointer when batch > 0.
 */
int mla_kv_append(const void* new_kv, void* kv_cache, const int32_t* block_table,
                  const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t num_pages,
                  int32_t max_pages_per_seq, hipStream_t stream);

/* The same for the GQA caches: new_k, new_v bf16 [batch, s_q, h_kv, 128]
 * (in) go to k_cache, v_cache bf16 [num_pages, 64, h_kv, 128] (in/out),
 * all h_kv groups of a token to the token's slot. 1 <= h_kv <= 4096. */
int gqa_kv_append(const void* new_k, const void* new_v, void* k_cache, void* v_cache,
                  const int32_t* block_table, const int32_t* cache_seqlens, int32_t batch,
                  int32_t s_q, int32_t h_kv, int32_t num_pages, int32_t max_pages_per_seq,
                  hipStream_t stream);

/* ---- FP8 latent cache ----
 *
 * The pages name FP8 only as FlashAttention-3's low-precision mode
 * (FlashAttention (KO), "FlashAttention-3 (2024)"); the format here is this
 * library's: per cached token, 576 OCP E4M3 codes (sign, 4 exponent bits
 * with bias 7, 3 mantissa bits; largest finite value 448; no infinities)
 * and one fp32 scale, value = e4m3(code) * scale, in two arrays:
 *   kv_codes   uint8 [num_pages, 64, 576]  (16-byte aligned)
 *   kv_scales  fp32  [num_pages, 64]       (4-byte aligned)
 * Quantising a bf16 row x: amax = max |x|; scale = the smallest power of
 * two not below the fp32 quotient amax / 448, at least 2^-126 (1 for an
 * all-zero row), a power-of-two scale as in the OCP microscaling formats;
 * code = the E4M3 value nearest to clamp(x / scale, -448, 448), ties to
 * even (x / scale is exact). Half the bytes of the bf16 cache (580 against
 * 1152 per token).
 */

/* MLA decode over an FP8 latent cache: as mla_decode, with V = the first
 * 512 dequantised columns. The plan comes from mla_decode_plan_fp8. The
 * scales are expected to be powers of two (as mla_kv_quantize_fp8 writes
 * them): with more than 32 query rows (s_q *
 * h_q) the pages are dequantised to bf16 values code * scale before the
 * products, which is exact for such scales (any other scale is rounded to
 * bf16 there; mla_check_fp8_scales finds such scales in a cache written by
 * other means). Errors as for mla_decode, plus MLA_ERR_NULL_ARG for
 * kv_scales = NULL and MLA_ERR_BAD_SHAPE for a misaligned kv_scales. */
int mla_decode_fp8(const void* q, const void* kv_codes, const float* kv_scales,
                   const int32_t* block_table, const int32_t* cache_seqlens, int32_t batch,
                   int32_t s_q, int32_t h_q, int32_t num_pages, int32_t max_pages_per_seq,
                   float softmax_scale, int32_t causal, const int32_t* sched_metadata,
                   const int32_t* num_splits, void* workspace, size_t workspace_bytes, void* out,
                   float* lse, hipStream_t stream);

/* Paged KV append into an FP8 cache: each of the s_q new tokens' bf16 rows
 * (new_kv [batch, s_q, 576]) is quantised into its slot (same slot rule,
 * skips and errors as mla_kv_append). Bit-exact: the codes and the scale
 * are what the rule above gives in fp32. */
int mla_kv_append_fp8(const void* new_kv, void* kv_codes, float* kv_scales,
                      const int32_t* block_table, const int32_t* cache_seqlens, int32_t batch,
                      int32_t s_q, int32_t num_pages, int32_t max_pages_per_seq,
                      hipStream_t stream);

/* Quantise n_rows bf16 latent rows (kv_rows [n_rows, 576], e.g. a whole
 * cache [num_pages, 64, 1, 576]) into kv_codes [n_rows, 576] and kv_scales
 * [n_rows] row for row. Errors: MLA_ERR_BAD_SHAPE for n_rows < 0 or
 * misaligned arrays, MLA_ERR_UNSUPPORTED past 2^31 - 1 rows,
 * MLA_ERR_NULL_ARG for a NULL pointer when n_rows > 0. */
int mla_kv_quantize_fp8(const void* kv_rows, void* kv_codes, float* kv_scales, int64_t n_rows,
                        hipStream_t stream);

/* ---- GQLA: one set of group-indexed weights, two decode paths ----
 *
 * GQLA (GQLA review, "2. Motivation & Problem Statement" and Figure 2) keeps
 * MLA's latent cache row [c (512), k_rope (64)] but indexes the key and value
 * up-projections by KV group: W_UK^g and W_UV^g, bf16 [h_kv, 512, 128], with
 * query head h in group g = h / (h_q / h_kv). Group g's key for a token is
 * [c W_UK^g, k_rope] (192 wide) and its value c W_UV^g (128 wide); a query
 * row is [q_nope (128), q_rope (64)]. The same weights give two decode paths
 * ("1. Key Terms & Definitions"):
 *   - MQA-absorb: gqla_absorb_query, then mla_decode over the latent cache
 *     (scale 1/sqrt(192)), then gqla_absorb_output;
 *   - GQA: gqla_expand_kv once per cached token (at append time), then
 *     gqla_decode over the expanded per-group caches.
 * The two agree up to rounding. The products run on bf16 MFMA with fp32
 * accumulation; every product output is rounded to bf16 (nearest-even).
 * Weights are [group][latent column][output column], row-major.
 */

/* Expanded per-group K and V rows of cached tokens (GQA path).
 *
 *   kv_rows  bf16 [n_rows, 576] (in): latent rows, e.g. a whole cache
 *            [num_pages, 64, 1, 576] (n_rows = 64 * num_pages) or the new
 *            tokens of an append [batch, s_q, 576]
 *   w_uk     bf16 [h_kv, 512, 128] (in); w_uv bf16 [h_kv, 512, 128] (in)
 *   k_rows   bf16 [n_rows, h_kv, 192] (out): [c W_UK^g, k_rope]
 *   v_rows   bf16 [n_rows, h_kv, 128] (out): c W_UV^g
 * A cache expanded page for page keeps the page layout of gqla_decode's
 * caches. Errors: MLA_ERR_BAD_SHAPE for n_rows < 0, h_kv outside 1..4096 or
 * unaligned tensors; MLA_ERR_UNSUPPORTED for n_rows > 2^31 - 1;
 * MLA_ERR_NULL_ARG for a NULL pointer when n_rows > 0. */
int gqla_expand_kv(const void* kv_rows, const void* w_uk, const void* w_uv, void* k_rows,
                   void* v_rows, int64_t n_rows, int32_t h_kv, hipStream_t stream);

/* Absorbed queries (MQA-absorb path): q_absorbed[n, h] =
 * [q_nope[n, h] W_UK^g^T, q_rope[n, h]], so that q_absorbed . latent row =
 * q . (group g's key).
 *
 *   q           bf16 [n_tokens, h_q, 192] (in), e.g. [batch, s_q, h_q, 192]
 *   w_uk        bf16 [h_kv, 512, 128] (in)
 *   q_absorbed  bf16 [n_tokens, h_q, 576] (out): mla_decode's q
 * Errors: MLA_ERR_BAD_SHAPE for n_tokens < 0, h_q < 1, h_kv < 1,
 * h_q % h_kv != 0 or unaligned tensors; MLA_ERR_UNSUPPORTED for h_kv > 65535
 * or n_tokens * h_q / h_kv near 2^31; MLA_ERR_NULL_ARG for a NULL pointer
 * when n_tokens > 0. */
int gqla_absorb_query(const void* q, const void* w_uk, void* q_absorbed, int32_t n_tokens,
                      int32_t h_q, int32_t h_kv, hipStream_t stream);

/* Output of the MQA-absorb path: out[n, h] = o_latent[n, h] W_UV^g.
 *
 *   o_latent  bf16 [n_tokens, h_q, 512] (in): mla_decode's out
 *   w_uv      bf16 [h_kv, 512, 128] (in)
 *   out       bf16 [n_tokens, h_q, 128] (out)
 * Errors as for gqla_absorb_query. */
int gqla_absorb_output(const void* o_latent, const void* w_uv, void* out, int32_t n_tokens,
                       int32_t h_q, int32_t h_kv, hipStream_t stream);

/* Decode on the GQA path over expanded caches (gqla_expand_kv's layout).
 *
 *   q        bf16 [batch, s_q, h_q, 192]
 *   k_cache  bf16 [num_pages, 64, h_kv, 192]
 *   v_cache  bf16 [num_pages, 64, h_kv, 128]
 *   out      bf16 [batch, s_q, h_q, 128] (out); lse fp32 [batch, s_q, h_q]
 *   softmax_scale multiplies the full 192-wide q.k (1/sqrt(192))
 * The plan comes from mla_decode_plan with the same h_kv and
 * head_dim_v = 128 (as for gqa_decode). Other arguments, preconditions and
 * errors as for gqa_decode. */
int gqla_decode(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_table, const int32_t* cache_seqlens, int32_t batch,
                int32_t s_q, int32_t h_q, int32_t h_kv, int32_t num_pages,
                int32_t max_pages_per_seq, float softmax_scale, int32_t causal,
                const int32_t* sched_metadata, const int32_t* num_splits, void* workspace,
                size_t workspace_bytes, void* out, float* lse, hipStream_t stream);

/* The plan's schedule computed on the host from host-resident lengths, for
 * checking the schedule on a machine without a GPU. num_workers, the
 * metadata layout and num_splits are exactly those mla_decode_plan would
 * write for the same arguments on a device with `num_cus` compute units.
 * seqlens_host, sched_metadata_host, num_splits_host and info are host
 * pointers. */
int mla_decode_plan_host(const int32_t* seqlens_host, int32_t batch, int32_t s_q, int32_t h_q,
                         int32_t h_kv, int32_t head_dim_v, int32_t num_cus,
                         int32_t* sched_metadata_host, int32_t* num_splits_host,
                         mla_plan_info* info);

/* Debug check of the device-side preconditions above, for callers that
 * want to validate a block table and lengths before a decode call (an
 * out-of-range page there is an out-of-bounds read). One small kernel on
 * `stream` reads cache_seqlens[0 .. batch) and, for each sequence whose
 * length is valid, block_table[b, j] for j < ceil(L_b / 64) (row stride
 * max_pages_per_seq), and writes status (device, int32 [4], 4-byte aligned,
 * no initialisation needed):
 *   status[0] = number of violations: lengths outside [0, 64 * max_pages_per_seq]
 *               plus used entries outside [0, num_pages);
 *   status[1] = sequence of the first violation in (b, j) order, or -1;
 *   status[2] = its page index j, or -1 when the length itself is invalid
 *               (0 when there is no violation);
 *   status[3] = the offending value (the length or the page id), else 0.
 * Pages of a sequence with an invalid length are not checked.
 * Errors: MLA_ERR_NULL_ARG for status = NULL, or a NULL table when batch > 0;
 * MLA_ERR_BAD_SHAPE for batch < 0, num_pages < 1, max_pages_per_seq < 1 or a
 * misaligned status. */
int mla_check_pages(const int32_t* block_table, const int32_t* cache_seqlens, int32_t batch,
                    int32_t num_pages, int32_t max_pages_per_seq, int32_t* status,
                    hipStream_t stream);

/* Debug check of an FP8 cache's per-token scales (the format above):
 * mla_decode_fp8 dequantises exactly only scales that are positive normal
 * powers of two, which is what mla_kv_quantize_fp8 writes; a cache filled
 * by other means can be checked with this call. One workgroup reads the n
 * fp32 scales at kv_scales and writes status int32[4] on the device:
 * [number of scales that are not positive normal powers of two, index of
 * the first such scale as two words (low, high; -1 when none), its fp32
 * bits (0 when none)]. Enqueued on `stream`; nothing is synchronised, and
 * the status needs no initialisation.
 * Errors: MLA_ERR_NULL_ARG for status = NULL, or kv_scales = NULL with
 * n > 0; MLA_ERR_BAD_SHAPE for n < 0 or a misaligned pointer. */
int mla_check_fp8_scales(const float* kv_scales, int64_t n, int32_t* status,
                         hipStream_t stream);

/* Profiling hook: while set, every mla_decode / gqa_decode call records the
 * HIP event `start` on its stream right before its main decode kernel and
 * `stop` right after it (before any merge kernel), so a caller can time that
 * kernel alone. Both are hipEvent_t handles; NULL clears the hook. Process-
 * wide and not thread-safe: meant for benchmarks, not for serving. */
void mla_profile_events(void* start, void* stop);

/* A short English text for a return code (static storage). */
const char* mla_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H_ */
