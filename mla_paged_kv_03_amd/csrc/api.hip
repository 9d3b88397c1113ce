// C interface: argument checks, launch geometry and kernel launches.
// Every check runs before anything is enqueued.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/mla_decode.h"
#include "kernels.h"
#include "schedule.h"

// Scratch of mla_decode_noalloc: the plan's metadata, its slot prefix and
// the fp32 split partials, in one static device array (one copy per GPU,
// held until the process ends). Host code never passes `scratch` itself to
// a kernel: its name on the host is only a handle, and the device address
// comes from hipGetSymbolAddress (noalloc_scratch below).
constexpr size_t NOALLOC_META_BYTES = (size_t)512 << 10;
constexpr size_t NOALLOC_SPLIT_BYTES = (size_t)512 << 10;
constexpr size_t NOALLOC_WS_BYTES = (size_t)136 << 20;
constexpr size_t NOALLOC_BYTES = NOALLOC_META_BYTES + NOALLOC_SPLIT_BYTES + NOALLOC_WS_BYTES;
static __device__ __align__(256) char scratch[NOALLOC_BYTES];

namespace {

constexpr int MLA_D = 576, MLA_DV = 512;  // latent row: 512 latent + 64 rope
constexpr int GQA_D = 128, GQA_DV = 128;
// GQLA widths: latent d_c, rope d_r, per-group key (no-rope) d_h and value d_v
constexpr int GQLA_DC = 512, GQLA_DR = 64, GQLA_DH = 128, GQLA_DVG = 128;
constexpr int GQLA_DQ = GQLA_DH + GQLA_DR;  // query and expanded key width (192)
constexpr int MAX_DEVICES = 64;
int g_cu_count[MAX_DEVICES];  // 0 = not queried yet
hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;  // mla_profile_events

int device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev >= 0 && dev < MAX_DEVICES && g_cu_count[dev] > 0) {
    *cus = g_cu_count[dev];
    return MLA_OK;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return MLA_ERR_HIP;
  if (dev >= 0 && dev < MAX_DEVICES) g_cu_count[dev] = n;
  *cus = n;
  return MLA_OK;
}

struct Geom {
  bool gqa;
  int B, T, H, G, D, DV;
  int M;      // query rows per KV head
  int nw;     // row groups of 16 rows per workgroup (1, 2 or 4)
  int nrb;    // row blocks per KV head
  int RB;     // row blocks per worker (all KV heads)
  // latent cache with 128 or more rows per KV head: the workers are those
  // of 128-row workgroups; the bf16 decode runs one 128-row block per
  // workgroup (nrb128 of them per worker), the FP8 decode keeps its 64-row
  // blocks (nrb of them per worker) over the same workers
  bool big;
  int nrb128;
  int fix;    // overhead units per piece of a sequence in the plan (schedule.h)
  int W;      // workers
  int TH;
  int max_slots;
  size_t meta_bytes, split_bytes, ws_bytes, lse_offset;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// fp8: the geometry of the FP8 latent decode, whose workgroups hold 64
// rows at any row count (its plan comes from mla_decode_plan_fp8)
int make_geom(int B, int T, int H, int G, int DV, int cus, Geom* g, bool fp8 = false) {
  if (B < 0 || T < 1 || H < 1 || G < 1 || H % G != 0) return MLA_ERR_BAD_SHAPE;
  if ((int64_t)T * H > (1 << 20)) return MLA_ERR_UNSUPPORTED;
  memset(g, 0, sizeof(*g));
  if (DV == MLA_DV) {
    if (G != 1) return MLA_ERR_UNSUPPORTED;
    g->gqa = false;
    g->D = MLA_D;
  } else if (DV == GQA_DV) {
    g->gqa = true;
    g->D = GQA_D;
  } else {
    return MLA_ERR_UNSUPPORTED;
  }
  g->B = B; g->T = T; g->H = H; g->G = G; g->DV = DV;
  g->M = T * H / G;
  g->nw = g->M <= 16 ? 1 : g->M <= 32 ? 2 : 4;
  const int rows = 16 * g->nw;
  g->nrb = (g->M + rows - 1) / rows;
  g->RB = G * g->nrb;
  g->big = !g->gqa && g->M >= 128 && !fp8;
  g->nrb128 = (g->M + 127) / 128;
  g->fix = g->big ? sched::FIX_LATENT128 : sched::FIX_DEFAULT;
  // one workgroup per CU for the latent cache (two 72 KiB page buffers);
  // the GQA pages are 32 KiB, so two workgroups share a CU
  const int per_cu = g->gqa ? 2 : 1;
  int W = cus * per_cu / (g->big ? g->nrb128 : g->RB);
  if (W >= 8) W -= W % 8;
  if (W < 1) W = 1;
  g->W = W;
  g->TH = T * H;
  g->max_slots = 2 * (W - 1);
  g->meta_bytes = ((size_t)sched::HDR + (size_t)W * sched::REC + (size_t)B + 1) * sizeof(int32_t);
  g->split_bytes = ((size_t)B + 1) * sizeof(int32_t);
  const size_t o_bytes = (size_t)g->max_slots * g->TH * DV * sizeof(float);
  const size_t l_bytes = (size_t)g->max_slots * g->TH * sizeof(float);
  g->lse_offset = align256(o_bytes);
  g->ws_bytes = g->max_slots ? g->lse_offset + l_bytes : 0;
  return MLA_OK;
}

void fill_info(const Geom& g, mla_plan_info* info) {
  info->num_workers = g.W;
  info->row_blocks = g.RB;
  info->max_split_slots = g.max_slots;
  info->reserved = 0;
  info->metadata_bytes = g.meta_bytes;
  info->num_splits_bytes = g.split_bytes;
  info->workspace_bytes = g.ws_bytes;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Pointer and value checks that need no device query.
int check_decode_args(bool gqa, const void* q, const void* k, const void* v,
                      const int32_t* block_table, const int32_t* seqlens, int num_pages,
                      int max_pages, float scale, int causal, const int32_t* meta,
                      const int32_t* splits, const void* out, const float* lse) {
  if (!q || !k || (gqa && !v) || !block_table || !seqlens || !meta || !splits || !out || !lse)
    return MLA_ERR_NULL_ARG;
  if (num_pages < 1 || max_pages < 1) return MLA_ERR_BAD_SHAPE;
  if (!(scale == scale) || isinf(scale)) return MLA_ERR_BAD_SHAPE;
  if (causal != 0 && causal != 1) return MLA_ERR_BAD_SHAPE;
  if (!aligned16(q) || !aligned16(k) || (v && !aligned16(v)) || !aligned16(out))
    return MLA_ERR_BAD_SHAPE;
  return MLA_OK;
}

int run_decode(int B, int T, int H, int G, int DV, int kind, const void* q, const void* k,
               const void* v, const float* kscale,
               const int32_t* block_table, const int32_t* seqlens, int num_pages,
               int max_pages, float scale, int causal, const int32_t* meta,
               const int32_t* splits, void* ws, size_t ws_bytes, void* out, float* lse,
               hipStream_t st) {
  Geom g;
  int rc, cus = 0;
  const bool fp8 = kind == mla::KIND_MLA_FP8;
  if ((rc = make_geom(B, T, H, G, DV, 1, &g, fp8)) != MLA_OK) return rc;
  if (B == 0) return MLA_OK;  // nothing to read or write (buffers may be empty)
  if ((rc = check_decode_args(g.gqa, q, k, v, block_table, seqlens, num_pages, max_pages, scale,
                              causal, meta, splits, out, lse)) != MLA_OK)
    return rc;
  if (kind == mla::KIND_MLA_FP8 && (!kscale || ((uintptr_t)kscale & 3)))
    return kscale ? MLA_ERR_BAD_SHAPE : MLA_ERR_NULL_ARG;
  if ((rc = device_cus(&cus)) != MLA_OK) return rc;
  make_geom(B, T, H, G, DV, cus, &g, fp8);
  if (g.ws_bytes) {
    if (!ws) return MLA_ERR_NULL_ARG;
    if (ws_bytes < g.ws_bytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
    if (((uintptr_t)ws & 255) != 0) return MLA_ERR_BAD_SHAPE;
  }

  mla::DecodeArgs a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.kscale = kscale;
  a.block_table = block_table;
  a.seqlens = seqlens;
  a.meta = meta;
  a.slots = splits;
  a.part_o = (float*)ws;
  a.part_lse = ws ? (float*)((char*)ws + g.lse_offset) : nullptr;
  a.out = (uint16_t*)out;
  a.lse = lse;
  a.B = g.B; a.T = g.T; a.H = g.H; a.G = g.G; a.bt_stride = max_pages;
  a.M = g.M; a.nrb = g.nrb; a.W = g.W;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.causal = causal;
  if (g_prof_start && hipEventRecord(g_prof_start, st) != hipSuccess) return MLA_ERR_HIP;
  hipError_t e;
  if (g.big && kind == mla::KIND_MLA) {
    a.nrb = g.nrb128;
    e = mla::launch_decode128_kernel(a, g.W * g.nrb128, st);
  } else {
    e = mla::launch_decode_kernel(a, g.nw, kind, g.W * g.RB, st);
  }
  if (e != hipSuccess) return MLA_ERR_HIP;
  if (g_prof_stop && hipEventRecord(g_prof_stop, st) != hipSuccess) return MLA_ERR_HIP;
  if (g.max_slots > 0) {
    mla::CombineArgs c;
    c.meta = meta;
    c.W = g.W;
    c.G = g.G;
    c.part_o = a.part_o;
    c.part_lse = a.part_lse;
    c.slots = splits;
    c.out = a.out;
    c.lse = lse;
    c.B = g.B; c.R = g.TH; c.DV = g.DV;
    // Sequences of equal length would each reach about W / B + 2 workers:
    // from 16 partials on the merge keeps four rows in flight per wave,
    // from 48 on it merges chunks of about 8 first (two launches)
    const int est = g.W / g.B + 2;
    c.Z = est >= 48 ? std::min((est + 7) / 8, 32) : 1;
    c.wide = est >= 16;
    c.level = 0;
    c.chunk_o = a.part_o;
    c.chunk_lse = a.part_lse;
    if (mla::launch_combine_kernel(c, st) != hipSuccess) return MLA_ERR_HIP;
  }
  return MLA_OK;
}

// Device address of this GPU's copy of `scratch`, looked up once per device
// (with that device current) and kept.
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];

int noalloc_scratch(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= MAX_DEVICES) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MLA_OK;
}

// Shared checks and launch of the paged KV append (both cache shapes).
int append_common(const void* src0, const void* src1, void* dst0, void* dst1,
                  const int32_t* block_table, const int32_t* cache_seqlens, int32_t batch,
                  int32_t s_q, size_t row_bytes, int32_t num_pages, int32_t max_pages_per_seq,
                  hipStream_t stream) {
  if (batch < 0 || s_q < 1 || num_pages < 0 || max_pages_per_seq < 0) return MLA_ERR_BAD_SHAPE;
  if ((int64_t)batch * s_q > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
  if (batch == 0) return MLA_OK;
  if (!src0 || !dst0 || !block_table || !cache_seqlens) return MLA_ERR_NULL_ARG;
  if (src1 && !dst1) return MLA_ERR_NULL_ARG;
  if (!aligned16(src0) || !aligned16(dst0) || (src1 && (!aligned16(src1) || !aligned16(dst1))))
    return MLA_ERR_BAD_SHAPE;
  mla::AppendArgs a;
  a.src0 = (const char*)src0;
  a.src1 = (const char*)src1;
  a.dst0 = (char*)dst0;
  a.dst1 = (char*)dst1;
  a.block_table = block_table;
  a.seqlens = cache_seqlens;
  a.row_bytes = row_bytes;
  a.B = batch;
  a.T = s_q;
  a.bt_stride = max_pages_per_seq;
  a.num_pages = num_pages;
  return mla::launch_kv_append(a, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// Head counts of the GQLA projections.
int gqla_heads(int32_t n_tokens, int32_t h_q, int32_t h_kv) {
  if (n_tokens < 0 || h_q < 1 || h_kv < 1 || h_q % h_kv != 0) return MLA_ERR_BAD_SHAPE;
  if (h_kv > 65535 || (int64_t)n_tokens * (h_q / h_kv) > 0x7fffffffLL - 128)
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

}  // namespace

extern "C" {

namespace {
int make_plan(const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t h_q,
              int32_t h_kv, int32_t head_dim_v, bool fp8, int32_t* sched_metadata,
              int32_t* num_splits, mla_plan_info* info, hipStream_t stream) {
  if (!info) return MLA_ERR_NULL_ARG;
  int cus = 0, rc;
  Geom g;
  if ((rc = make_geom(batch, s_q, h_q, h_kv, head_dim_v, 1, &g, fp8)) != MLA_OK) return rc;
  if ((sched_metadata || num_splits) &&
      (!sched_metadata || !num_splits || (batch > 0 && !cache_seqlens)))
    return MLA_ERR_NULL_ARG;
  if ((rc = device_cus(&cus)) != MLA_OK) return rc;
  make_geom(batch, s_q, h_q, h_kv, head_dim_v, cus, &g, fp8);
  fill_info(g, info);
  if (!sched_metadata && !num_splits) return MLA_OK;
  if (mla::launch_plan_kernel(cache_seqlens, batch, g.W, g.TH, g.G, g.DV, g.fix, sched_metadata,
                              num_splits, stream) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}
}  // namespace

int mla_decode_plan(const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t h_q,
                    int32_t h_kv, int32_t head_dim_v, int32_t* sched_metadata,
                    int32_t* num_splits, mla_plan_info* info, hipStream_t stream) {
  return make_plan(cache_seqlens, batch, s_q, h_q, h_kv, head_dim_v, false, sched_metadata,
                   num_splits, info, stream);
}

int mla_decode_plan_fp8(const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t h_q,
                        int32_t* sched_metadata, int32_t* num_splits, mla_plan_info* info,
                        hipStream_t stream) {
  return make_plan(cache_seqlens, batch, s_q, h_q, 1, MLA_DV, true, sched_metadata, num_splits,
                   info, stream);
}

int mla_decode(const void* q, const void* kv_cache, const int32_t* block_table,
               const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t h_q,
               int32_t num_pages, int32_t max_pages_per_seq, float softmax_scale,
               int32_t causal, const int32_t* sched_metadata, const int32_t* num_splits,
               void* workspace, size_t workspace_bytes, void* out, float* lse,
               hipStream_t stream) {
  return run_decode(batch, s_q, h_q, 1, MLA_DV, mla::KIND_MLA, q, kv_cache, nullptr, nullptr, block_table, cache_seqlens, num_pages,
                    max_pages_per_seq, softmax_scale, causal, sched_metadata, num_splits,
                    workspace, workspace_bytes, out, lse, stream);
}

int mla_decode_noalloc(const void* q, const void* kv_cache, const int32_t* block_table,
                       const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t h_q,
                       int32_t num_pages, int32_t max_pages_per_seq, float softmax_scale,
                       int32_t causal, void* out, float* lse, hipStream_t stream) {
  Geom g;
  int rc, cus = 0;
  if ((rc = make_geom(batch, s_q, h_q, 1, MLA_DV, 1, &g)) != MLA_OK) return rc;
  if (batch == 0) return MLA_OK;
  // the plan buffers live in the scratch: check the caller's pointers now,
  // with stand-ins for those, so that nothing is enqueued on an error
  const int32_t* stand_in = cache_seqlens;
  if ((rc = check_decode_args(false, q, kv_cache, nullptr, block_table, cache_seqlens, num_pages,
                              max_pages_per_seq, softmax_scale, causal, stand_in, stand_in, out,
                              lse)) != MLA_OK)
    return rc;
  if ((rc = device_cus(&cus)) != MLA_OK) return rc;
  make_geom(batch, s_q, h_q, 1, MLA_DV, cus, &g);
  if (g.meta_bytes > NOALLOC_META_BYTES || g.split_bytes > NOALLOC_SPLIT_BYTES ||
      g.ws_bytes > NOALLOC_WS_BYTES)
    return MLA_ERR_SCRATCH_LIMIT;
  void* base = nullptr;
  if ((rc = noalloc_scratch(&base)) != MLA_OK) return rc;
  int32_t* meta = (int32_t*)base;
  int32_t* splits = (int32_t*)((char*)base + NOALLOC_META_BYTES);
  void* ws = (char*)base + NOALLOC_META_BYTES + NOALLOC_SPLIT_BYTES;
  // the plan kernel rewrites every word the decode and merge read, so
  // nothing in the scratch needs clearing between calls
  if (mla::launch_plan_kernel(cache_seqlens, batch, g.W, g.TH, g.G, g.DV, g.fix, meta, splits,
                              stream) != hipSuccess)
    return MLA_ERR_HIP;
  return run_decode(batch, s_q, h_q, 1, MLA_DV, mla::KIND_MLA, q, kv_cache, nullptr, nullptr,
                    block_table, cache_seqlens, num_pages, max_pages_per_seq, softmax_scale,
                    causal, meta, splits, ws, NOALLOC_WS_BYTES, out, lse, stream);
}

int gqa_decode(const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_table, const int32_t* cache_seqlens, int32_t batch,
               int32_t s_q, int32_t h_q, int32_t h_kv, int32_t num_pages,
               int32_t max_pages_per_seq, float softmax_scale, int32_t causal,
               const int32_t* sched_metadata, const int32_t* num_splits, void* workspace,
               size_t workspace_bytes, void* out, float* lse, hipStream_t stream) {
  return run_decode(batch, s_q, h_q, h_kv, GQA_DV, mla::KIND_GQA, q, k_cache, v_cache, nullptr, block_table, cache_seqlens, num_pages,
                    max_pages_per_seq, softmax_scale, causal, sched_metadata, num_splits,
                    workspace, workspace_bytes, out, lse, stream);
}

int attn_combine(const float* o_partial, const float* lse_partial, const int32_t* num_splits,
                 int32_t batch, int32_t rows_per_batch, int32_t dv, void* out, float* lse,
                 hipStream_t stream) {
  if (batch < 0 || rows_per_batch < 0 || dv < 8 || dv > 1024 || dv % 8) return MLA_ERR_BAD_SHAPE;
  if (batch == 0 || rows_per_batch == 0) return MLA_OK;
  if (!o_partial || !lse_partial || !num_splits || !out || !lse) return MLA_ERR_NULL_ARG;
  if (!aligned16(o_partial) || !aligned16(out)) return MLA_ERR_BAD_SHAPE;
  mla::CombineArgs c;
  c.meta = nullptr;  // the caller's own slot prefix: no plan to check
  c.W = 0;
  c.G = 0;
  c.part_o = o_partial;
  c.part_lse = lse_partial;
  c.slots = num_splits;
  c.out = (uint16_t*)out;
  c.lse = lse;
  c.B = batch; c.R = rows_per_batch; c.DV = dv;
  c.level = 0;  // one pass: the caller's partials are never overwritten
  c.Z = 1;
  c.wide = 0;
  c.chunk_o = nullptr;
  c.chunk_lse = nullptr;
  return mla::launch_combine_kernel(c, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_kv_append(const void* new_kv, void* kv_cache, const int32_t* block_table,
                  const int32_t* cache_seqlens, int32_t batch, int32_t s_q, int32_t num_pages,
                  int32_t max_pages_per_seq, hipStream_t stream) {
  return append_common(new_kv, nullptr, kv_cache, nullptr, block_table, cache_seqlens, batch,
                       s_q, (size_t)MLA_D * 2, num_pages, max_pages_per_seq, stream);
}

int gqa_kv_append(const void* new_k, const void* new_v, void* k_cache, void* v_cache,
                  const int32_t* block_table, const int32_t* cache_seqlens, int32_t batch,
                  int32_t s_q, int32_t h_kv, int32_t num_pages, int32_t max_pages_per_seq,
                  hipStream_t stream) {
  if (h_kv < 1 || h_kv > 4096) return MLA_ERR_BAD_SHAPE;
  if (batch > 0 && (!new_v || !v_cache)) return MLA_ERR_NULL_ARG;
  return append_common(new_k, new_v, k_cache, v_cache, block_table, cache_seqlens, batch, s_q,
                       (size_t)h_kv * GQA_D * 2, num_pages, max_pages_per_seq, stream);
}

int mla_decode_fp8(const void* q, const void* kv_codes, const float* kv_scales,
                   const int32_t* block_table, const int32_t* cache_seqlens, int32_t batch,
                   int32_t s_q, int32_t h_q, int32_t num_pages, int32_t max_pages_per_seq,
                   float softmax_scale, int32_t causal, const int32_t* sched_metadata,
                   const int32_t* num_splits, void* workspace, size_t workspace_bytes, void* out,
                   float* lse, hipStream_t stream) {
  return run_decode(batch, s_q, h_q, 1, MLA_DV, mla::KIND_MLA_FP8, q, kv_codes, nullptr,
                    kv_scales, block_table, cache_seqlens, num_pages, max_pages_per_seq,
                    softmax_scale, causal, sched_metadata, num_splits, workspace,
                    workspace_bytes, out, lse, stream);
}

int mla_kv_append_fp8(const void* new_kv, void* kv_codes, float* kv_scales,
                      const int32_t* block_table, const int32_t* cache_seqlens, int32_t batch,
                      int32_t s_q, int32_t num_pages, int32_t max_pages_per_seq,
                      hipStream_t stream) {
  if (batch < 0 || s_q < 1 || num_pages < 0 || max_pages_per_seq < 0) return MLA_ERR_BAD_SHAPE;
  if ((int64_t)batch * s_q > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
  if (batch == 0) return MLA_OK;
  if (!new_kv || !kv_codes || !kv_scales || !block_table || !cache_seqlens) return MLA_ERR_NULL_ARG;
  if (!aligned16(new_kv) || !aligned16(kv_codes) || ((uintptr_t)kv_scales & 3))
    return MLA_ERR_BAD_SHAPE;
  mla::QuantArgs a = {};
  a.src = (const uint16_t*)new_kv;
  a.codes = (uint8_t*)kv_codes;
  a.scales = kv_scales;
  a.block_table = block_table;
  a.seqlens = cache_seqlens;
  a.B = batch; a.T = s_q; a.bt_stride = max_pages_per_seq; a.num_pages = num_pages;
  return mla::launch_quantize_fp8(a, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_kv_quantize_fp8(const void* kv_rows, void* kv_codes, float* kv_scales, int64_t n_rows,
                        hipStream_t stream) {
  if (n_rows < 0) return MLA_ERR_BAD_SHAPE;
  if (n_rows > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
  if (n_rows == 0) return MLA_OK;
  if (!kv_rows || !kv_codes || !kv_scales) return MLA_ERR_NULL_ARG;
  if (!aligned16(kv_rows) || !aligned16(kv_codes) || ((uintptr_t)kv_scales & 3))
    return MLA_ERR_BAD_SHAPE;
  mla::QuantArgs a = {};
  a.src = (const uint16_t*)kv_rows;
  a.codes = (uint8_t*)kv_codes;
  a.scales = kv_scales;
  a.B = (int)n_rows; a.T = 1;
  return mla::launch_quantize_fp8(a, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int gqla_decode(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_table, const int32_t* cache_seqlens, int32_t batch,
                int32_t s_q, int32_t h_q, int32_t h_kv, int32_t num_pages,
                int32_t max_pages_per_seq, float softmax_scale, int32_t causal,
                const int32_t* sched_metadata, const int32_t* num_splits, void* workspace,
                size_t workspace_bytes, void* out, float* lse, hipStream_t stream) {
  return run_decode(batch, s_q, h_q, h_kv, GQLA_DVG, mla::KIND_GQA_ROPE, q, k_cache, v_cache,
                    nullptr, block_table,
                    cache_seqlens, num_pages, max_pages_per_seq, softmax_scale, causal,
                    sched_metadata, num_splits, workspace, workspace_bytes, out, lse, stream);
}

int gqla_absorb_query(const void* q, const void* w_uk, void* q_absorbed, int32_t n_tokens,
                      int32_t h_q, int32_t h_kv, hipStream_t stream) {
  int rc;
  if ((rc = gqla_heads(n_tokens, h_q, h_kv)) != MLA_OK) return rc;
  if (n_tokens == 0) return MLA_OK;
  if (!q || !w_uk || !q_absorbed) return MLA_ERR_NULL_ARG;
  if (!aligned16(q) || !aligned16(w_uk) || !aligned16(q_absorbed)) return MLA_ERR_BAD_SHAPE;
  const int hpg = h_q / h_kv;
  mla::GemmArgs a = {};
  a.a = (const uint16_t*)q;
  a.inner = hpg;
  a.a_outer = (int64_t)h_q * GQLA_DQ; a.a_inner = GQLA_DQ; a.a_batch = (int64_t)hpg * GQLA_DQ;
  a.b = (const uint16_t*)w_uk;  // [c][i]: row c of W_UK^g is column c of the product
  a.b_batch = (int64_t)GQLA_DC * GQLA_DH; a.ldb = GQLA_DH; a.b_kn = 0;
  a.c = (uint16_t*)q_absorbed;
  a.c_outer = (int64_t)h_q * (GQLA_DC + GQLA_DR); a.c_inner = GQLA_DC + GQLA_DR;
  a.c_batch = (int64_t)hpg * (GQLA_DC + GQLA_DR);
  a.M = n_tokens * hpg; a.N = GQLA_DC; a.K = GQLA_DH; a.batches = h_kv;
  a.rope = 1; a.rope_a_off = GQLA_DH; a.rope_c_off = GQLA_DC;  // q_rope passes through
  return mla::launch_gemm(a, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int gqla_absorb_output(const void* o_latent, const void* w_uv, void* out, int32_t n_tokens,
                       int32_t h_q, int32_t h_kv, hipStream_t stream) {
  int rc;
  if ((rc = gqla_heads(n_tokens, h_q, h_kv)) != MLA_OK) return rc;
  if (n_tokens == 0) return MLA_OK;
  if (!o_latent || !w_uv || !out) return MLA_ERR_NULL_ARG;
  if (!aligned16(o_latent) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_BAD_SHAPE;
  const int hpg = h_q / h_kv;
  mla::GemmArgs a = {};
  a.a = (const uint16_t*)o_latent;
  a.inner = hpg;
  a.a_outer = (int64_t)h_q * GQLA_DC; a.a_inner = GQLA_DC; a.a_batch = (int64_t)hpg * GQLA_DC;
  a.b = (const uint16_t*)w_uv;  // [c][j]: K rows, N contiguous
  a.b_batch = (int64_t)GQLA_DC * GQLA_DVG; a.ldb = GQLA_DVG; a.b_kn = 1;
  a.c = (uint16_t*)out;
  a.c_outer = (int64_t)h_q * GQLA_DVG; a.c_inner = GQLA_DVG; a.c_batch = (int64_t)hpg * GQLA_DVG;
  a.M = n_tokens * hpg; a.N = GQLA_DVG; a.K = GQLA_DC; a.batches = h_kv;
  return mla::launch_gemm(a, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int gqla_expand_kv(const void* kv_rows, const void* w_uk, const void* w_uv, void* k_rows,
                   void* v_rows, int64_t n_rows, int32_t h_kv, hipStream_t stream) {
  if (n_rows < 0 || h_kv < 1 || h_kv > 4096) return MLA_ERR_BAD_SHAPE;
  if (n_rows > 0x7fffffffLL) return MLA_ERR_UNSUPPORTED;
  if (n_rows == 0) return MLA_OK;
  if (!kv_rows || !w_uk || !w_uv || !k_rows || !v_rows) return MLA_ERR_NULL_ARG;
  if (!aligned16(kv_rows) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(k_rows) ||
      !aligned16(v_rows))
    return MLA_ERR_BAD_SHAPE;
  static_assert(GQLA_DH == 128 && GQLA_DVG == 128 && GQLA_DC == 512, "expansion kernel widths");
  mla::ExpandArgs a = {};
  a.a = (const uint16_t*)kv_rows;
  a.M = n_rows;
  a.G = h_kv;
  // workgroups: about one per CU, in slices of 8 (one per XCD) per pair of
  // groups (a workgroup expands two groups)
  int cus = 0;
  if (device_cus(&cus) != MLA_OK) return MLA_ERR_HIP;
  const int pairs = (h_kv + 1) / 2;
  const int per_pair = (cus + pairs - 1) / pairs;
  a.n_slices = 8 * ((per_pair + 7) / 8);
  // K: group g's columns 0..127 of each expanded row, plus the shared rope
  a.w = (const uint16_t*)w_uk;
  a.c = (uint16_t*)k_rows;
  a.c_outer = (int64_t)h_kv * GQLA_DQ; a.c_batch = GQLA_DQ;
  a.rope = 1; a.rope_c_off = GQLA_DH;
  if (mla::launch_expand(a, stream) != hipSuccess) return MLA_ERR_HIP;
  // V
  a.w = (const uint16_t*)w_uv;
  a.c = (uint16_t*)v_rows;
  a.c_outer = (int64_t)h_kv * GQLA_DVG; a.c_batch = GQLA_DVG;
  a.rope = 0;
  return mla::launch_expand(a, stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_decode_plan_host(const int32_t* seqlens_host, int32_t batch, int32_t s_q, int32_t h_q,
                         int32_t h_kv, int32_t head_dim_v, int32_t num_cus,
                         int32_t* sched_metadata_host, int32_t* num_splits_host,
                         mla_plan_info* info) {
  if (!info) return MLA_ERR_NULL_ARG;
  if (num_cus < 1) return MLA_ERR_BAD_SHAPE;
  Geom g;
  int rc;
  if ((rc = make_geom(batch, s_q, h_q, h_kv, head_dim_v, num_cus, &g)) != MLA_OK) return rc;
  fill_info(g, info);
  if (!sched_metadata_host && !num_splits_host) return MLA_OK;
  if (!sched_metadata_host || !num_splits_host || (batch > 0 && !seqlens_host))
    return MLA_ERR_NULL_ARG;
  sched::host_plan(seqlens_host, batch, g.W, g.TH, g.G, g.DV, g.fix, sched_metadata_host,
                   num_splits_host);
  return MLA_OK;
}

int mla_check_pages(const int32_t* block_table, const int32_t* cache_seqlens, int32_t batch,
                    int32_t num_pages, int32_t max_pages_per_seq, int32_t* status,
                    hipStream_t stream) {
  if (!status) return MLA_ERR_NULL_ARG;
  if (batch < 0 || num_pages < 1 || max_pages_per_seq < 1) return MLA_ERR_BAD_SHAPE;
  if (batch > 0 && (!block_table || !cache_seqlens)) return MLA_ERR_NULL_ARG;
  if (((uintptr_t)status & 3) != 0) return MLA_ERR_BAD_SHAPE;
  if (mla::launch_check_pages(block_table, cache_seqlens, batch, num_pages, max_pages_per_seq,
                              status, stream) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_check_fp8_scales(const float* kv_scales, int64_t n, int32_t* status, hipStream_t stream) {
  if (!status) return MLA_ERR_NULL_ARG;
  if (n < 0) return MLA_ERR_BAD_SHAPE;
  if (n > 0 && !kv_scales) return MLA_ERR_NULL_ARG;
  if (((uintptr_t)status & 3) != 0 || ((uintptr_t)kv_scales & 3) != 0) return MLA_ERR_BAD_SHAPE;
  if (mla::launch_check_fp8_scales(kv_scales, n, status, stream) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

void mla_profile_events(void* start, void* stop) {
  g_prof_start = (hipEvent_t)start;
  g_prof_stop = (hipEvent_t)stop;
}

const char* mla_status_string(int code) {
  switch (code) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL_ARG: return "a required pointer is NULL";
    case MLA_ERR_BAD_SHAPE: return "invalid shape, alignment or argument value";
    case MLA_ERR_UNSUPPORTED: return "head dimensions or sizes not supported by this build";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than the plan requires";
    case MLA_ERR_HIP: return "HIP runtime error";
    case MLA_ERR_SCRATCH_LIMIT: return "the call needs more than the library's static scratch";
  }
  return "unknown status";
}

}  // extern "C"
