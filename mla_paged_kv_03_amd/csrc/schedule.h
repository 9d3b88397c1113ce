// Split-KV schedule: how the pages of a variable-length batch are spread
// over a fixed set of workgroups ("workers").
//
// FlashAttention (KO), section "FlashAttention-2 (2023)", credits better
// parallelism and work partitioning across the GPU; the FlashMLA blog
// ("기술 기반") asks for efficient variable-length handling. A worker pays
// `fix` overhead units (loading the queries, writing the result) for every
// piece of a sequence it processes, and one unit per 64-token page. The plan:
//   1. Sequence b costs p_b + fix units if one worker takes it whole; with
//      T the batch's total of that cost, it is cut into
//      k_b = clamp(round((p_b + fix) * W / T), 1, p_b) pieces: its share
//      of the W workers.
//   2. Sequence b is laid out as k_b blocks, each `fix` overhead units
//      followed by its pages (the first p_b % k_b blocks one page more than
//      the others); the blocks of the whole batch are concatenated and the
//      line is cut into W equal contiguous ranges of `chunk` units.
// So a worker that starts a piece of a split sequence finds that piece's
// overhead at the start of its range, and a batch of equal sequences splits
// into equal pieces exactly on the block boundaries. A sequence whose pages
// fall into several ranges is split; each piece writes a partial result
// that a log-sum-exp merge finishes. `fix` is part of the plan
// (FIX_LATENT128 for the 128-row latent decode, whose queries and output
// weigh several pages, FIX_DEFAULT otherwise) and is recorded in the plan's
// signature, with T.
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
enum : int { H_MAGIC = 0, H_W = 1, H_B = 2, H_ROWS = 3, H_G = 4, H_DV = 5, H_FIX = 6, H_COST = 7 };

SCHED_HD void write_header(int32_t* hdr, int W, int B, int rows, int G, int DV, int fix,
                           int32_t cost) {
  hdr[H_MAGIC] = PLAN_MAGIC;
  hdr[H_W] = W;
  hdr[H_B] = B;
  hdr[H_ROWS] = rows;
  hdr[H_G] = G;
  hdr[H_DV] = DV;
  hdr[H_FIX] = fix;
  hdr[H_COST] = cost;
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
// cost of sequence b taken whole (step 1); T is their sum over the batch
SCHED_HD int seq_cost(int32_t L, int fix) { return seq_pages(L) + fix; }
// number of pieces (blocks) of a sequence: its share of the workers, at
// least one and at most one per page
SCHED_HD int seq_pieces(int32_t L, int fix, int32_t T, int W) {
  const int p = seq_pages(L);
  if (p == 0 || T <= 0) return 1;
  // round(cost * W / T); in 32-bit arithmetic whenever it fits (a 64-bit
  // division is far slower on the GPU; both give the same quotient)
  const uint64_t num = 2 * (uint64_t)seq_cost(L, fix) * (uint64_t)W + (uint64_t)T;
  const uint64_t den = 2 * (uint64_t)T;
  const uint64_t k = (num >> 32) == 0 && (den >> 32) == 0 ? (uint32_t)num / (uint32_t)den
                                                          : num / den;
  return k < 1 ? 1 : (k > (uint64_t)p ? p : (int)k);
}
// units of a sequence on the line (step 2): every block's overhead and pages
SCHED_HD int seq_units(int32_t L, int fix, int32_t T, int W) {
  const int p = seq_pages(L);
  return p + fix * seq_pieces(L, fix, T, W);
}
// Pages of a sequence that lie before its unit offset x (0 <= x <= units):
// the overhead units of a block count as lying before the block's pages.
// (All in 32 bits: a sequence's units, like the whole line, fit in int32.)
// (with the sequence's pages p >= 1 and its pieces n = seq_pieces given)
SCHED_HD int pages_before_pn(int p, int n, int fix, int32_t x) {
  const int q = p / n, r = p % n;  // blocks 0 .. r - 1 hold q + 1 pages, the rest q
  const int big = fix + q + 1, small = fix + q, xr = r * big;
  int i, off, before;
  if (x < xr) {
    i = x / big;
    off = x - i * big;
    before = i * (q + 1);
  } else {
    i = r + (x - xr) / small;
    off = (x - xr) - (i - r) * small;
    before = r * (q + 1) + (i - r) * q;
  }
  if (i >= n) return p;
  const int bp = i < r ? q + 1 : q;
  const int in = off - fix;
  return before + (in < 0 ? 0 : (in > bp ? bp : in));
}
SCHED_HD int pages_before(int32_t L, int fix, int32_t T, int W, int32_t x) {
  const int p = seq_pages(L);
  if (p == 0) return 0;
  return pages_before_pn(p, seq_pieces(L, fix, T, W), fix, x);
}

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

// Units per worker: at least one more than a block's overhead, so that a
// range inside a split sequence always holds one of its pages.
SCHED_HD int chunk_units(int32_t total_units, int W, int fix) {
  const int c = (total_units + W - 1) / W;
  return c > fix ? c : fix + 1;
}

// The rest of worker_record, with its first and last sequences bs and be
// (the sequences holding unit offsets lo and hi - 1) already found.
// pbs, nbs (pbe, nbe): pages and pieces (seq_pieces) of bs (be).
SCHED_HD void record_of(int w, int chunk, int64_t lo, int64_t hi, int bs, int be, int pbs, int nbs,
                        int pbe, int nbe, const int32_t* prefix, int fix, int32_t* rec) {
  const int ps = pbs == 0 ? 0 : pages_before_pn(pbs, nbs, fix, (int32_t)(lo - prefix[bs]));
  const int pe = pbe == 0 ? 0 : pages_before_pn(pbe, nbe, fix, (int32_t)(hi - prefix[be]));
  // the worker holding the sequence's first page (its first block opens
  // with the overhead units)
  const int first_w = (prefix[bs] + fix) / chunk;
  rec[R_B_START] = bs;
  rec[R_P_START] = ps;
  rec[R_B_END] = be;
  rec[R_P_END] = pe;
  rec[R_SPLIT0] = w > first_w ? w - first_w : 0;
  rec[R_OWNS_FIRST] = prefix[bs] == lo ? 1 : 0;
  rec[R_LO] = (int32_t)lo;
  rec[R_HI] = (int32_t)hi;
}

// Record of worker w. prefix has B + 1 entries (prefix[B] = total units of
// the line); T is the batch's cost from step 1.
SCHED_HD void worker_record(int w, int W, const int32_t* prefix, const int32_t* seqlens,
                            int B, int fix, int32_t T, int32_t* rec) {
  const int32_t C = prefix[B];
  const int chunk = chunk_units(C, W, fix);
  const int64_t lo = (int64_t)w * chunk;
  if (lo >= C) {
    rec[R_B_START] = 0; rec[R_P_START] = 0; rec[R_B_END] = -1; rec[R_P_END] = 0;
    rec[R_SPLIT0] = 0; rec[R_OWNS_FIRST] = 0; rec[R_LO] = C; rec[R_HI] = C;
    return;
  }
  const int64_t hi = (lo + chunk < C) ? lo + chunk : C;
  const int bs = find_seq(prefix, B, lo);
  const int be = find_seq(prefix, B, hi - 1);
  record_of(w, chunk, lo, hi, bs, be, seq_pages(seqlens[bs]), seq_pieces(seqlens[bs], fix, T, W),
            seq_pages(seqlens[be]), seq_pieces(seqlens[be], fix, T, W), prefix, fix, rec);
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

// Number of workers that process pages of sequence b (1 for an empty one):
// those holding its first page, its last unit (a page: every block ends with
// pages) and every range between, each of which holds a page since a range
// is longer than a block's overhead.
SCHED_HD int seq_split_count(int b, int W, const int32_t* prefix, const int32_t* seqlens, int B,
                             int fix) {
  if (seq_pages(seqlens[b]) == 0) return 1;
  const int chunk = chunk_units(prefix[B], W, fix);
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

// The whole plan on the host, in the order the plan kernel computes it:
// header, prefix of line units, worker records, slot prefix (B + 1 entries).
inline void host_plan(const int32_t* seqlens, int B, int W, int rows, int G, int DV, int fix,
                      int32_t* meta, int32_t* splits) {
  int64_t T = 0;
  for (int b = 0; b < B; ++b) T += seq_cost(seqlens[b], fix);
  write_header(meta, W, B, rows, G, DV, fix, (int32_t)T);
  int32_t* prefix = unit_prefix(meta, W);
  prefix[0] = 0;
  for (int b = 0; b < B; ++b) prefix[b + 1] = prefix[b] + seq_units(seqlens[b], fix, (int32_t)T, W);
  for (int w = 0; w < W; ++w)
    worker_record(w, W, prefix, seqlens, B, fix, (int32_t)T, records(meta) + (size_t)w * REC);
  int32_t acc = 0;
  for (int b = 0; b < B; ++b) {
    splits[b] = acc;
    acc += seq_slots(b, W, prefix, seqlens, B, fix);
  }
  splits[B] = acc;
}

}  // namespace sched
