// Split-KV schedule: how the pages of a variable-length batch are spread
// over a fixed set of workgroups ("workers").
//
// FlashAttention (KO), section "FlashAttention-2 (2023)", credits better
// parallelism and work partitioning across the GPU; the FlashMLA blog
// ("기술 기반") asks for efficient variable-length handling. Here the work
// of sequence b is `fix` overhead units (loading its queries, writing its
// result) followed by one unit per 64-token page; the units of the whole
// batch are concatenated and cut into num_workers equal contiguous ranges of
// `chunk` units. A sequence whose pages fall into several ranges is split;
// each piece writes a partial result that a log-sum-exp merge finishes.
// `fix` is part of the plan (FIX_LATENT128 for the 128-row latent decode,
// whose per-sequence queries and output weigh several pages, FIX_DEFAULT
// otherwise) and is recorded in the plan's signature.
//
// Every function here is plain arithmetic usable on the host (for the
// host-side checker) and on the device (for the plan kernel).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define SCHED_HD __host__ __device__ inline
#else
#define SCHED_HD inline
#endif

namespace sched {

constexpr int PAGE = 64;
constexpr int FIX_DEFAULT = 2;
constexpr int FIX_LATENT128 = 6;
constexpr int REC = 8;  // int32 per worker record

// The metadata opens with a signature of the geometry the plan was made for
// (HDR int32 words); the worker records follow it, then the unit prefix.
// The decode and merge kernels compare it with their own geometry before
// they index any record or slot, and leave every output untouched when a
// plan made for another batch, worker count, row count, KV head count or
// value width is passed in.
constexpr int HDR = 8;
constexpr int32_t PLAN_MAGIC = 0x4D4C4150;  // "PALM" in memory order
enum : int { H_MAGIC = 0, H_W = 1, H_B = 2, H_ROWS = 3, H_G = 4, H_DV = 5, H_FIX = 6 };

SCHED_HD void write_header(int32_t* hdr, int W, int B, int rows, int G, int DV, int fix) {
  hdr[H_MAGIC] = PLAN_MAGIC;
  hdr[H_W] = W;
  hdr[H_B] = B;
  hdr[H_ROWS] = rows;
  hdr[H_G] = G;
  hdr[H_DV] = DV;
  hdr[H_FIX] = fix;
  hdr[7] = 0;
}

// Records of the workers, and the unit prefix, inside the metadata.
SCHED_HD const int32_t* records(const int32_t* meta) { return meta + HDR; }
SCHED_HD int32_t* records(int32_t* meta) { return meta + HDR; }
SCHED_HD int32_t* unit_prefix(int32_t* meta, int W) { return meta + HDR + (size_t)W * REC; }

// Worker record layout (int32 x REC).
enum : int {
  R_B_START = 0,    // first sequence touched
  R_P_START = 1,    // first page of R_B_START
  R_B_END = 2,      // last sequence touched (inclusive); < R_B_START when idle
  R_P_END = 3,      // one past the last page of R_B_END
  R_SPLIT0 = 4,     // split index of this worker's piece of R_B_START
  R_OWNS_FIRST = 5, // 1 if this worker holds the first unit of R_B_START
  R_LO = 6,         // unit range [lo, hi)
  R_HI = 7
};

SCHED_HD int seq_pages(int32_t L) { return L > 0 ? (L + PAGE - 1) / PAGE : 0; }
SCHED_HD int seq_units(int32_t L, int fix) { return seq_pages(L) + fix; }

// Largest b in [0, B) with prefix[b] <= u (prefix strictly increasing,
// prefix[0] = 0 <= u).
SCHED_HD int find_seq(const int32_t* prefix, int B, int64_t u) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= u) lo = mid; else hi = mid - 1;
  }
  return lo;
}

SCHED_HD int chunk_units(int32_t total_units, int W) {
  int c = (total_units + W - 1) / W;
  return c > 0 ? c : 1;
}

// Record of worker w. prefix has B + 1 entries (prefix[B] = total units).
SCHED_HD void worker_record(int w, int W, const int32_t* prefix, const int32_t* seqlens,
                            int B, int fix, int32_t* rec) {
  const int32_t C = prefix[B];
  const int chunk = chunk_units(C, W);
  const int64_t lo = (int64_t)w * chunk;
  if (lo >= C) {
    rec[R_B_START] = 0; rec[R_P_START] = 0; rec[R_B_END] = -1; rec[R_P_END] = 0;
    rec[R_SPLIT0] = 0; rec[R_OWNS_FIRST] = 0; rec[R_LO] = C; rec[R_HI] = C;
    return;
  }
  const int64_t hi = (lo + chunk < C) ? lo + chunk : C;
  const int bs = find_seq(prefix, B, lo);
  const int be = find_seq(prefix, B, hi - 1);
  int64_t ps = lo - prefix[bs] - fix;
  if (ps < 0) ps = 0;
  const int ne = seq_pages(seqlens[be]);
  int64_t pe = hi - prefix[be] - fix;
  if (pe < 0) pe = 0;
  if (pe > ne) pe = ne;
  const int first_w = (prefix[bs] + fix) / chunk;
  rec[R_B_START] = bs;
  rec[R_P_START] = (int32_t)ps;
  rec[R_B_END] = be;
  rec[R_P_END] = (int32_t)pe;
  rec[R_SPLIT0] = w > first_w ? w - first_w : 0;
  rec[R_OWNS_FIRST] = prefix[bs] == lo ? 1 : 0;
  rec[R_LO] = (int32_t)lo;
  rec[R_HI] = (int32_t)hi;
}

// Pages [p0, p1) of sequence b (with npg pages) that worker record rec
// covers, given the worker's first and last sequences bs and be. Clamped to
// the sequence's current page count, so a plan made for longer lengths never
// sends a worker past the pages the lengths reach (the result is then not
// the attention of those lengths, but nothing outside them is read).
SCHED_HD void page_range(const int32_t* rec, int b, int bs, int be, int npg, int* p0, int* p1) {
  int lo = b == bs ? rec[R_P_START] : 0;
  int hi = b == be ? rec[R_P_END] : npg;
  hi = hi < npg ? hi : npg;
  lo = lo < 0 ? 0 : lo;
  *p0 = lo;
  *p1 = hi;
}

// Number of workers that process pages of sequence b (1 for an empty one).
SCHED_HD int seq_split_count(int b, int W, const int32_t* prefix, const int32_t* seqlens, int B,
                             int fix) {
  if (seq_pages(seqlens[b]) == 0) return 1;
  const int chunk = chunk_units(prefix[B], W);
  const int first = (prefix[b] + fix) / chunk;
  const int last = (prefix[b + 1] - 1) / chunk;
  return last - first + 1;
}

// Partial-result slots of sequence b: none when one worker finishes it.
SCHED_HD int seq_slots(int b, int W, const int32_t* prefix, const int32_t* seqlens, int B,
                       int fix) {
  const int n = seq_split_count(b, W, prefix, seqlens, B, fix);
  return n > 1 ? n : 0;
}

}  // namespace sched
