// Latent-cache decode at 128 query rows per workgroup (MLA with 128 or more
// query rows per KV head: the 128-head DeepSeek-V3 shapes and their
// multi-token variants), on v_mfma_f32_32x32x16_bf16.
//
// Method as in decode_kernels.hip (FlashAttention (KO): tiling, online
// softmax, one fused kernel; paged cache per PagedAttention with 64-token
// pages; the GQLA review's MQA-absorb shape). What differs is the tile:
//   * Four waves, one per SIMD, each owning 32 query rows, so that both
//     products run on 32x32x16 MFMA tiles (on gfx950 these sustain about
//     0.97 of the bf16 peak from one wave per SIMD) and every K or V
//     fragment read from LDS feeds 32 rows instead of 16.
//   * A page is copied into LDS once per 128 rows (once per CU for a
//     128-head step). Each wave copies 16 of the page's 64 rows
//     (global_load_lds_dwordx4, 18 copies of 1 KiB) for the next page while
//     its score MFMAs for the current page run; one barrier per page.
//   * Scores are computed transposed, S^T[key][row] = K Q^T: lane l holds
//     row l % 32 and 16 keys of each 32-key block, so a row's max and sums
//     are in-lane reductions plus one swap with lane l ^ 32. The score
//     registers, rounded to bf16, are directly the P^T operand of
//     O^T[dv][row] += V^T P^T, whose V^T operand comes from the same LDS page
//     by transposed reads (ds_read_b64_tr_b16), so every cache byte crosses
//     HBM once.
//   * O^T (512 x 32 fp32 per wave) stays in the 256 accumulation registers;
//     Q (32 rows x 576) stays in 144 registers for the whole sequence.
//   * Softmax: each row keeps a fixed reference m, the max of the first
//     page on which the row sees a key, so O is only ever touched by MFMA.
//     If a later page exceeds it by more than 2^REF_LIMIT, the workgroup
//     reruns the range twice: once for the exact row maxima (scores only),
//     then against them.
#include "decode_device.h"
#include "schedule.h"

namespace mla {

namespace {

constexpr int R128_WAVES = 4;
constexpr int R128_KC = 36;                  // 16-column steps of the 576-wide scores
constexpr int R128_NT = 16;                  // 32-column tiles of the 512-wide output
constexpr int R128_NDMA = 18;                // 1 KiB page copies per wave and page
constexpr int R128_KBLK = 32 * 1152;         // LDS bytes of 32 page rows
constexpr int R128_PFK = 4;                  // score-operand prefetch distance (steps)
constexpr int R128_PFV = 3;                  // value-operand prefetch distance (steps)
// page copies issued among the 72 score MFMAs (the rest among the 64 P V ones)
constexpr int R128_DMA_QK = 18;

// copy index issued after score step st, or -1
constexpr int qk_dma_slot(int st) {
  return R128_DMA_QK == 18 ? (st % 4 == 2 ? st / 4 : -1)
                           : (st % 8 == 4 && st / 8 < R128_DMA_QK ? st / 8 : -1);
}
// copy index issued after P V step st, or -1
constexpr int pv_dma_slot(int st) {
  return R128_DMA_QK == 18 ? -1
                           : (st % 7 == 3 && R128_DMA_QK + st / 7 < 18 ? R128_DMA_QK + st / 7 : -1);
}

enum : int { PASS_FIRST_REF = 0, PASS_MAX_ONLY = 1, PASS_PRESET_REF = 2 };

template <int V>
using pass_tag = std::integral_constant<int, V>;


// Score MFMAs with their accumulators in VGPRs (the 256 accumulation
// registers hold O). Written as asm because the compiler, given both as
// builtins, placed the scores in accumulation registers and moved O out.
// The asm carries the hazard wait states the compiler does not see: two
// before the MFMA (a VALU write of an operand), and scores_ready below
// before any VALU instruction touches the results.
__device__ __forceinline__ f32x16 mfma32_v_zero(const bf16x8& a, const bf16x8& b) {
  f32x16 d;
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void mfma32_v_acc(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// A 16-pass MFMA's VGPR results may be read (and its SrcC registers
// rewritten) by VALU instructions only some 20 wait states after it issues.
__device__ __forceinline__ void scores_ready(f32x16& s0, f32x16& s1) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s0), "+v"(s1));
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Scalar loads from wave-uniform addresses, issued together and waited for
// in the same statement: one memory round trip for all of them. Each block
// opens with one wait state after a possible VALU write of the address
// registers; the results are early-clobber, so no result register doubles as
// an address still to be read.

// The first six words at p in one round trip.
__device__ __forceinline__ void sload6(const int32_t* p, int (&v)[6]) {
  int a0, a1, a2, a3, a4, a5;
  asm volatile(
      "s_nop 0\n\ts_load_dword %0, %6, 0x0\n\ts_load_dword %1, %6, 0x4\n\t"
      "s_load_dword %2, %6, 0x8\n\ts_load_dword %3, %6, 0xc\n\ts_load_dword %4, %6, 0x10\n\t"
      "s_load_dword %5, %6, 0x14\n\ts_waitcnt lgkmcnt(0)"
      : "=&s"(a0), "=&s"(a1), "=&s"(a2), "=&s"(a3), "=&s"(a4), "=&s"(a5)
      : "s"(p)
      : "memory");
  v[0] = a0; v[1] = a1; v[2] = a2; v[3] = a3; v[4] = a4; v[5] = a5;
}
// A sequence's length *p, its slot range *q and *(q + 1), and the
// block-table entries *r0 and *r1 (its first two pages in this range), in
// one round trip.
__device__ __forceinline__ void sload_seq(const int32_t* p, const int32_t* q, const int32_t* r0,
                                          const int32_t* r1, int& x, int& y0, int& y1, int& z0,
                                          int& z1) {
  asm volatile(
      "s_nop 0\n\ts_load_dword %0, %5, 0x0\n\ts_load_dword %1, %6, 0x0\n\t"
      "s_load_dword %2, %6, 0x4\n\ts_load_dword %3, %7, 0x0\n\ts_load_dword %4, %8, 0x0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(x), "=&s"(y0), "=&s"(y1), "=&s"(z0), "=&s"(z1)
      : "s"(p), "s"(q), "s"(r0), "s"(r1)
      : "memory");
}

// *p and *q in one round trip
__device__ __forceinline__ void sload_2(const int32_t* p, const int32_t* q, int& x, int& y) {
  asm volatile("s_nop 0\n\ts_load_dword %0, %2, 0x0\n\ts_load_dword %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(x), "=&s"(y)
               : "s"(p), "s"(q)
               : "memory");
}

// Raw buffer descriptor of n bytes from p (no stride, 32-bit data format):
// loads at offsets >= n return zeros and read no memory.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* p, uint32_t n) {
  const uintptr_t u = (uintptr_t)p;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(u >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)n);
  r[3] = 0x00020000;
  return r;
}

// One 1 KiB HBM -> LDS copy through a buffer descriptor: lane l's 16 bytes
// at voff land at LDS byte lds + LOFF + 16 l (zeros past the descriptor's
// range). m0 is formed inside the asm from one base register and the
// compile-time offset, so the copies of a page need no register per copy.
// Same wait states as dma16: five after a VALU write of a descriptor SGPR,
// one between the write of m0 and the copy.
template <int LOFF>
__device__ __forceinline__ void dma16_buf(uint32_t lds, i32x4 rsrc, uint32_t voff) {
  asm volatile("s_nop 4\n\ts_add_u32 m0, %0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc), "i"(LOFF)
               : "memory", "m0");
}

}  // namespace

__global__ __launch_bounds__(64 * R128_WAVES) void decode128_kernel(DecodeArgs a) {
  using LY = Layout<KIND_MLA>;
  static_assert(LY::K_PITCH == 1152 && LY::TILE == 64 * 1152, "latent page layout");
  __shared__ __attribute__((aligned(1024))) char lds[2 * LY::TILE];
  lds_char* const lds_p = LDS_PTR(char, lds);
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds_p;

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;   // query row within the wave
  const int hf = lane >> 5;  // which half of each MFMA's 16 k-slots the lane holds

  int w, rb;
  decode_block_id_xcd(blockIdx.x, a.W, a.nrb, w, rb);

  // Wave-uniform values come in by scalar loads. First the plan's signature
  // (its six words in one round trip): a plan made for another geometry
  // leaves every output untouched, and its buffer may not even hold this
  // worker's record, which is read only after the signature matches.
  static_assert(sched::H_MAGIC < 6 && sched::H_W < 6 && sched::H_B < 6 && sched::H_ROWS < 6 &&
                    sched::H_G < 6 && sched::H_DV < 6,
                "the signature words compared here are its first six");
  int hw[6];
  sload6(uniform_ptr(a.meta), hw);
  if ((hw[sched::H_MAGIC] != sched::PLAN_MAGIC) | (hw[sched::H_W] != a.W) |
      (hw[sched::H_B] != a.B) | (hw[sched::H_ROWS] != a.T * a.H) | (hw[sched::H_G] != a.G) |
      (hw[sched::H_DV] != LY::DV))
    return;
  const int32_t* rec = uniform_ptr(sched::records(a.meta) + w * sched::REC);
  static_assert(sched::R_B_START < 6 && sched::R_B_END < 6 && sched::R_OWNS_FIRST < 6 &&
                    sched::R_SPLIT0 < 6 && sched::R_P_START < 6 && sched::R_P_END < 6,
                "the record words read here are its first six");
  int rw[6];
  sload6(rec, rw);
  const int bs = rw[sched::R_B_START];
  const int be = rw[sched::R_B_END];
  if (be < bs) return;
  const int owns_first = rw[sched::R_OWNS_FIRST];
  const int split0 = rw[sched::R_SPLIT0];
  const int p_start = rw[sched::R_P_START];
  const int p_end = rw[sched::R_P_END];

  const int TH = a.T * a.H;
  const bool scale_neg = a.scale_log2 < 0.f;
  const float scale_abs = fabsf(a.scale_log2);
  const int rho = rb * 128 + wave * 32 + n;  // output row within a sequence (t * H + h)
  const bool row_ok = rho < TH;
  const int t = row_ok ? rho / a.H : 0;

  // ---- per-lane LDS offsets inside a page buffer ----
  // A page lands as it lies in HBM (64 rows of 1152 bytes), with 16-byte
  // chunk c of row r at chunk c ^ row_xor(r) (an XOR below 8 keeps a chunk
  // inside its aligned group of 8, rope included). row_xor spreads both read
  // patterns over the LDS banks (rows 1152 bytes apart share a bank window
  // every second row): the score reads (16 lanes read one chunk of 16
  // consecutive rows) see distinct XOR values on the 8 even and the 8 odd
  // rows, and the transposed value reads (32 lanes read 4 chunks of 4
  // consecutive rows) see rows r and r + 2 one aligned group of 4 chunks
  // apart.
  auto row_xor = [](int r) { return 4 * ((r >> 1) & 1) + 2 * ((r >> 2) & 1) + ((r >> 3) & 1); };
  // Score operand A = K[key][16 columns]: lane l reads key 32kb + n, columns
  // 16c + 8hf .. +7, i.e. chunk 2c + hf of the row; four offsets (c % 4)
  // plus 128 (c / 4) cover every step (32kb leaves row_xor unchanged).
  uint32_t k_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) k_off[q] = n * 1152 + 16 * ((2 * q + hf) ^ row_xor(n));
  // Value operand A = V^T[32 columns][16 keys] by transposed reads: the
  // 16-lane group g reads 4 keys x 16 columns (lane j: key 4hf + j / 4,
  // columns 16(g & 1) + 4(j % 4) .. +3) and lane j receives column j's 4
  // keys. Read lo takes keys 32kb + 16s + 4hf + (0..3), read hi the same + 8
  // (whose row_xor differs in bit 0, hence its own offsets).
  const int g16 = lane >> 4, j16 = lane & 15;
  const int vrow = 4 * hf + (j16 >> 2);
  uint32_t v_off[2], v_off_hi[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = 4 * q + 2 * (g16 & 1) + ((j16 & 3) >> 1);
    v_off[q] = vrow * 1152 + 16 * (c ^ row_xor(vrow)) + 8 * (j16 & 1);
    v_off_hi[q] = (vrow + 8) * 1152 + 16 * (c ^ row_xor(vrow + 8)) + 8 * (j16 & 1);
  }

  // Page copies: wave w fills LDS rows 16w .. 16w + 15 of a page buffer
  // (18 KiB) with 18 copies of 1 KiB. Copy tt writes LDS units
  // 1152w + 64tt + lane (16 bytes each), i.e. row 16w + rr, chunk x with
  // 64tt + lane = 72rr + x; that chunk holds HBM chunk x ^ row_xor(rr) of
  // the row. Copies tt and tt + 9 lie exactly 8 rows apart, whose row_xor
  // differs in bit 0: the second nine use the first nine's offsets with
  // bit 4 flipped, through a descriptor 8 rows on.
  uint32_t dma_off[9];
  for (int tt = 0; tt < 9; ++tt) {
    const int u = 64 * tt + lane;
    const int rr = u / 72;
    const int x = u - 72 * rr;
    dma_off[tt] = (uint32_t)(wave * (16 * 1152) + rr * 1152 + 16 * (x ^ row_xor(rr)));
  }

  const int32_t* seqlens = uniform_ptr(a.seqlens);
  const int32_t* slots = uniform_ptr(a.slots);
  // The length, slot range and first two block-table entries of sequence b
  // (pages from p0 on) in one round trip. The indices are clamped into the
  // row, so the lookups stay inside the block table whatever the lengths
  // (they differ from p0 and p0 + 1 only where a length needs more pages
  // than a row holds); an entry past the sequence's pages is loaded but not
  // used.
  auto lookup = [&](int b, int p0, int& L, int& s0, int& s1, int& pg_a, int& pg_b) {
    const int32_t* bt = a.block_table + (size_t)b * a.bt_stride;
    const int pa = min(max(p0, 0), a.bt_stride - 1);
    const int pb = min(pa + 1, a.bt_stride - 1);
    sload_seq(seqlens + b, slots + b, uniform_ptr(bt + pa), uniform_ptr(bt + pb), L, s0, s1, pg_a,
              pg_b);
  };
  // Descriptors of a page's two halves of rows (rows 0..7 and 8..15 of each
  // wave's 16) holding its first nb bytes: copies past them return zeros
  // (finite values whose keys the mask drops) and read nothing, so every
  // wave issues the same copies on every page.
  auto make_rsrc = [&](int page, int nb, i32x4& lo, i32x4& hi) {
    const char* base = (const char*)a.k + (size_t)page * LY::TILE;
    lo = buffer_rsrc(base, (uint32_t)nb);
    hi = buffer_rsrc(base + 8 * 1152, (uint32_t)max(nb - 8 * 1152, 0));
  };
  // copy T (a literal, 0 .. 17) of this wave into the page buffer at LDS
  // byte BUF0
#define MLA_DMA_ONE(T, LO, HI, BUF0)                                              \
  dma16_buf<1024 * (T)>((BUF0) + wave * (16 * 1152), (T) < 9 ? (LO) : (HI),       \
                        (T) < 9 ? dma_off[(T) < 9 ? (T) : 0] : dma_off[(T) < 9 ? 0 : (T) - 9] ^ 16u)
#define MLA_DMA_ALL(LO, HI, BUF0)                                                                 \
  MLA_DMA_ONE(0, LO, HI, BUF0); MLA_DMA_ONE(1, LO, HI, BUF0); MLA_DMA_ONE(2, LO, HI, BUF0);     \
  MLA_DMA_ONE(3, LO, HI, BUF0); MLA_DMA_ONE(4, LO, HI, BUF0); MLA_DMA_ONE(5, LO, HI, BUF0);     \
  MLA_DMA_ONE(6, LO, HI, BUF0); MLA_DMA_ONE(7, LO, HI, BUF0); MLA_DMA_ONE(8, LO, HI, BUF0);     \
  MLA_DMA_ONE(9, LO, HI, BUF0); MLA_DMA_ONE(10, LO, HI, BUF0); MLA_DMA_ONE(11, LO, HI, BUF0);   \
  MLA_DMA_ONE(12, LO, HI, BUF0); MLA_DMA_ONE(13, LO, HI, BUF0); MLA_DMA_ONE(14, LO, HI, BUF0);  \
  MLA_DMA_ONE(15, LO, HI, BUF0); MLA_DMA_ONE(16, LO, HI, BUF0); MLA_DMA_ONE(17, LO, HI, BUF0)

  // whether the current sequence's first page went into buffer 0 before
  // the epilogue of the sequence ahead of it
  bool next_page = false;

  for (int b = bs; b <= be; ++b) {
    const int32_t* bt = a.block_table + (size_t)b * a.bt_stride;
    int L, s0, s1, pg_a, pg_b;
    lookup(b, b == bs ? p_start : 0, L, s0, s1, pg_a, pg_b);
    const bool page_issued = next_page;
    next_page = false;
    const int npg = sched::seq_pages(L);
    // the page range of schedule.h's page_range, from the record's words
    int p0 = b == bs ? p_start : 0;
    int p1 = b == be ? p_end : npg;
    p1 = min(p1, npg);
    p0 = max(p0, 0);
    const int nslots = s1 - s0;

    if (npg == 0) {
      if ((b > bs || owns_first) && row_ok) {
        uint16_t* o = a.out + ((size_t)b * TH + rho) * LY::DV;
#pragma unroll
        for (int tt = 0; tt < R128_NT; ++tt)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *(u32x2*)(o + 32 * tt + 8 * q + 4 * hf) = u32x2{0u, 0u};
        if (hf == 0) a.lse[(size_t)b * TH + rho] = -INFINITY;
      }
      continue;
    }
    if (p0 >= p1) continue;
    const int split = b == bs ? split0 : 0;

    // queries of this lane's row: B operand of the score MFMA, columns
    // 16c + 8hf .. +7 at step c; loaded once the first page's copies are in
    // flight, so that the two latencies overlap
    bf16x8 qf[R128_KC];
    auto load_q = [&]() {
      const uint16_t* qrow = a.q + ((size_t)b * TH + rho) * LY::D;
#pragma unroll
      for (int c = 0; c < R128_KC; ++c) {
        const u32x4 x = row_ok ? *(const u32x4*)(qrow + 16 * c + 8 * hf) : u32x4{0u, 0u, 0u, 0u};
        qf[c] = __builtin_bit_cast(bf16x8, x);
      }
    };
    // With a negative softmax scale the queries are negated (exactly: a sign
    // flip) and the scale's magnitude used, so scale * score keeps its value
    // and the row max is always a max of raw scores. The flip waits until
    // the first page has landed, so that the query loads overlap its copies.
    auto flip_q = [&]() {
      const uint32_t flip = scale_neg ? 0x80008000u : 0u;
#pragma unroll
      for (int c = 0; c < R128_KC; ++c)
        qf[c] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qf[c]) ^ flip);
    };
    const int vis = a.causal ? min(L - a.T + 1 + t, L) : L;
    // keys below this are visible to every row of the workgroup
    const int vis_all = a.causal ? L - a.T + 1 : L;

    // page j of this sequence: valid == false covers nothing (the copies
    // then move no data)
    auto page_rsrc_of = [&](int j, int page, bool valid, i32x4& lo, i32x4& hi) {
      make_rsrc(page, valid ? min(64, L - 64 * j) * 1152 : 0, lo, hi);
    };
    auto page_rsrc = [&](int j, bool valid, i32x4& lo, i32x4& hi) {
      page_rsrc_of(j, sload(uniform_ptr(bt + j)), valid, lo, hi);
    };

    f32x16 o[R128_NT];
    float m = -INFINITY, l = 0.f, lw = 0.f;

    // One pass over the pages [p0, p1) of sequence b.
    auto run_pass = [&](auto mode_tag) -> bool {
      constexpr int MODE = decltype(mode_tag)::value;
      if constexpr (MODE != PASS_MAX_ONLY) {
#pragma unroll
        for (int tt = 0; tt < R128_NT; ++tt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[tt][r] = 0.f;
        l = 0.f;
        lw = 0.f;
      }
      if constexpr (MODE != PASS_PRESET_REF) m = -INFINITY;
      bool over = false;

      if constexpr (MODE != PASS_FIRST_REF) {  // page p0 into buffer 0 (the first
                                              // pass finds it issued)
        i32x4 lo, hi;
        page_rsrc_of(p0, pg_a, true, lo, hi);
        MLA_DMA_ALL(lo, hi, lds0);
      }
      for (int j = p0; j < p1; ++j) {
        const int cur = (j - p0) & 1;
        const bool has_next = j + 1 < p1;
        i32x4 nlo, nhi;
        if (j == p0 && has_next)
          page_rsrc_of(j + 1, pg_b, true, nlo, nhi);
        else
          page_rsrc(has_next ? j + 1 : j, has_next, nlo, nhi);
        const uint32_t ndst = lds0 + (cur ^ 1) * LY::TILE;
        // this wave's copies of page j have landed; after the barrier every
        // wave's have, and every wave is done with page j - 1, whose buffer
        // the copies of page j + 1 refill
        wait_vm<0>();
        barrier();
        lds_char* const buf = lds_p + cur * LY::TILE;
        if constexpr (MODE == PASS_FIRST_REF) {
          if (j == p0) flip_q();
        }

        // ---- S^T = K Q^T for the page's two 32-key blocks ----
        auto k_frag = [&](int st) -> bf16x8 {
          const int c = st >> 1, kb = st & 1;
          return *(const __attribute__((address_space(3))) bf16x8*)(
              buf + k_off[c & 3] + 128 * (c >> 2) + kb * R128_KBLK);
        };
        f32x16 sc[2];
        bf16x8 kf[R128_PFK + 1];
#pragma unroll
        for (int st = 0; st < R128_PFK; ++st) kf[st] = k_frag(st);
        // 72 steps (c = st / 2 over the 576 columns, kb = st % 2), written
        // out so that each copy of the next page carries its LDS offset as a
        // literal
#define MLA_QK_STEP(ST)                                                                         \
  {                                                                                             \
    if ((ST) + R128_PFK < 2 * R128_KC)                                                          \
      kf[((ST) + R128_PFK) % (R128_PFK + 1)] = k_frag((ST) + R128_PFK);                         \
    if ((ST) < 2)                                                                               \
      sc[(ST) & 1] = mfma32_v_zero(kf[(ST) % (R128_PFK + 1)], qf[(ST) >> 1]);                   \
    else                                                                                        \
      mfma32_v_acc(sc[(ST) & 1], kf[(ST) % (R128_PFK + 1)], qf[(ST) >> 1]);                     \
    constexpr int T_ = qk_dma_slot(ST);                                                         \
    if constexpr (T_ >= 0) MLA_DMA_ONE(T_ < 0 ? 0 : T_, nlo, nhi, ndst);                        \
    mem_fence_compiler();                                                                       \
  }
        MLA_QK_STEP(0) MLA_QK_STEP(1) MLA_QK_STEP(2) MLA_QK_STEP(3) MLA_QK_STEP(4)
        MLA_QK_STEP(5) MLA_QK_STEP(6) MLA_QK_STEP(7) MLA_QK_STEP(8) MLA_QK_STEP(9)
        MLA_QK_STEP(10) MLA_QK_STEP(11) MLA_QK_STEP(12) MLA_QK_STEP(13) MLA_QK_STEP(14)
        MLA_QK_STEP(15) MLA_QK_STEP(16) MLA_QK_STEP(17) MLA_QK_STEP(18) MLA_QK_STEP(19)
        MLA_QK_STEP(20) MLA_QK_STEP(21) MLA_QK_STEP(22) MLA_QK_STEP(23) MLA_QK_STEP(24)
        MLA_QK_STEP(25) MLA_QK_STEP(26) MLA_QK_STEP(27) MLA_QK_STEP(28) MLA_QK_STEP(29)
        MLA_QK_STEP(30) MLA_QK_STEP(31) MLA_QK_STEP(32) MLA_QK_STEP(33) MLA_QK_STEP(34)
        MLA_QK_STEP(35) MLA_QK_STEP(36) MLA_QK_STEP(37) MLA_QK_STEP(38) MLA_QK_STEP(39)
        MLA_QK_STEP(40) MLA_QK_STEP(41) MLA_QK_STEP(42) MLA_QK_STEP(43) MLA_QK_STEP(44)
        MLA_QK_STEP(45) MLA_QK_STEP(46) MLA_QK_STEP(47) MLA_QK_STEP(48) MLA_QK_STEP(49)
        MLA_QK_STEP(50) MLA_QK_STEP(51) MLA_QK_STEP(52) MLA_QK_STEP(53) MLA_QK_STEP(54)
        MLA_QK_STEP(55) MLA_QK_STEP(56) MLA_QK_STEP(57) MLA_QK_STEP(58) MLA_QK_STEP(59)
        MLA_QK_STEP(60) MLA_QK_STEP(61) MLA_QK_STEP(62) MLA_QK_STEP(63) MLA_QK_STEP(64)
        MLA_QK_STEP(65) MLA_QK_STEP(66) MLA_QK_STEP(67) MLA_QK_STEP(68) MLA_QK_STEP(69)
        MLA_QK_STEP(70) MLA_QK_STEP(71)
#undef MLA_QK_STEP
        scores_ready(sc[0], sc[1]);

        // ---- mask, row max ----
        // register r of block kb holds key 64j + 32kb + 8(r / 4) + 4hf + r % 4;
        // keys past what the row sees get -inf (on the pages that have any),
        // by a sign mask rather than compares, so no scalar masks pile up
        if (64 * (j + 1) > vis_all) {
          const int d0 = 64 * j + 4 * hf - vis;  // key - vis, less the constant part
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const uint32_t keep = (uint32_t)((d0 + 32 * kb + 8 * (r >> 2) + (r & 3)) >> 31);
              sc[kb][r] = __uint_as_float((__float_as_uint(sc[kb][r]) & keep) |
                                          (0xff800000u & ~keep));
            }
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sc[kb][r]);
        {
          const uint32_t u = __float_as_uint(tmax);
          const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
          tmax = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1])) * scale_abs;
        }
        if constexpr (MODE == PASS_MAX_ONLY) {
          m = fmaxf(m, tmax);
          // the copies the P V steps would have issued
#define MLA_PV_DMA_ONLY(ST)                                                  \
  {                                                                          \
    constexpr int T_ = pv_dma_slot(ST);                                      \
    if constexpr (T_ >= 0) MLA_DMA_ONE(T_ < 0 ? 0 : T_, nlo, nhi, ndst);     \
  }
          MLA_PV_DMA_ONLY(0) MLA_PV_DMA_ONLY(1) MLA_PV_DMA_ONLY(2) MLA_PV_DMA_ONLY(3)
          MLA_PV_DMA_ONLY(4) MLA_PV_DMA_ONLY(5) MLA_PV_DMA_ONLY(6) MLA_PV_DMA_ONLY(7)
          MLA_PV_DMA_ONLY(8) MLA_PV_DMA_ONLY(9) MLA_PV_DMA_ONLY(10) MLA_PV_DMA_ONLY(11)
          MLA_PV_DMA_ONLY(12) MLA_PV_DMA_ONLY(13) MLA_PV_DMA_ONLY(14) MLA_PV_DMA_ONLY(15)
          MLA_PV_DMA_ONLY(16) MLA_PV_DMA_ONLY(17) MLA_PV_DMA_ONLY(18) MLA_PV_DMA_ONLY(19)
          MLA_PV_DMA_ONLY(20) MLA_PV_DMA_ONLY(21) MLA_PV_DMA_ONLY(22) MLA_PV_DMA_ONLY(23)
          MLA_PV_DMA_ONLY(24) MLA_PV_DMA_ONLY(25) MLA_PV_DMA_ONLY(26) MLA_PV_DMA_ONLY(27)
          MLA_PV_DMA_ONLY(28) MLA_PV_DMA_ONLY(29) MLA_PV_DMA_ONLY(30) MLA_PV_DMA_ONLY(31)
          MLA_PV_DMA_ONLY(32) MLA_PV_DMA_ONLY(33) MLA_PV_DMA_ONLY(34) MLA_PV_DMA_ONLY(35)
          MLA_PV_DMA_ONLY(36) MLA_PV_DMA_ONLY(37) MLA_PV_DMA_ONLY(38) MLA_PV_DMA_ONLY(39)
          MLA_PV_DMA_ONLY(40) MLA_PV_DMA_ONLY(41) MLA_PV_DMA_ONLY(42) MLA_PV_DMA_ONLY(43)
          MLA_PV_DMA_ONLY(44) MLA_PV_DMA_ONLY(45) MLA_PV_DMA_ONLY(46) MLA_PV_DMA_ONLY(47)
          MLA_PV_DMA_ONLY(48) MLA_PV_DMA_ONLY(49) MLA_PV_DMA_ONLY(50) MLA_PV_DMA_ONLY(51)
          MLA_PV_DMA_ONLY(52) MLA_PV_DMA_ONLY(53) MLA_PV_DMA_ONLY(54) MLA_PV_DMA_ONLY(55)
          MLA_PV_DMA_ONLY(56) MLA_PV_DMA_ONLY(57) MLA_PV_DMA_ONLY(58) MLA_PV_DMA_ONLY(59)
          MLA_PV_DMA_ONLY(60) MLA_PV_DMA_ONLY(61) MLA_PV_DMA_ONLY(62) MLA_PV_DMA_ONLY(63)
#undef MLA_PV_DMA_ONLY
          continue;
        }
        if constexpr (MODE == PASS_FIRST_REF) {
          if (m == -INFINITY) m = tmax;
          over = over || tmax > m + REF_LIMIT;
        }
        const float m_use = m == -INFINITY ? 0.f : m;

        // ---- weights exp2(scale * s - m): l sums them as computed (for the
        // LSE), lw as the P V MFMA receives them, rounded to bf16 (it divides
        // the output; a dot product with (1, 1) adds a rounded pair) ----
        bf16x8 pf[4];
        float psum = 0.f, wsum = 0.f;
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        typedef float f32x2_t __attribute__((ext_vector_type(2)));
        const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            u32x4 pk;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float pa = fast_exp2(__builtin_fmaf(sc[kb][8 * s + 2 * e], scale_abs, -m_use));
              const float pb = fast_exp2(__builtin_fmaf(sc[kb][8 * s + 2 * e + 1], scale_abs, -m_use));
              psum += pa + pb;
              const bf16x2_t w2 = __builtin_convertvector((f32x2_t){pa, pb}, bf16x2_t);
              wsum = __builtin_amdgcn_fdot2_f32_bf16(w2, ones, wsum, false);
              pk[e] = __builtin_bit_cast(uint32_t, w2);
            }
            pf[2 * kb + s] = __builtin_bit_cast(bf16x8, pk);
          }
        l += psum;
        lw += wsum;

        // ---- O^T += V^T P^T: step s4 = 2kb + s covers keys 32kb + 16s ..
        // +15, whose k-slots 8hf + i hold score registers 8s + i of block kb
        auto v_frag = [&](int st) -> bf16x8 {
          const int tt = st & 15, s4 = st >> 4;
          const int off = 128 * (tt >> 1) + (16 * s4) * 1152;
          const bf16x4 lo =
              __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(buf + v_off[tt & 1] + off));
          const bf16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(buf + v_off_hi[tt & 1] + off));
          return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        bf16x8 vf[R128_PFV + 1];
#pragma unroll
        for (int st = 0; st < R128_PFV; ++st) vf[st] = v_frag(st);
#define MLA_PV_STEP(ST)                                                                         \
  {                                                                                             \
    if ((ST) + R128_PFV < 4 * R128_NT)                                                          \
      vf[((ST) + R128_PFV) % (R128_PFV + 1)] = v_frag((ST) + R128_PFV);                         \
    o[(ST) & 15] = mfma32(vf[(ST) % (R128_PFV + 1)], pf[(ST) >> 4], o[(ST) & 15]);              \
    constexpr int T_ = pv_dma_slot(ST);                                                         \
    if constexpr (T_ >= 0) MLA_DMA_ONE(T_ < 0 ? 0 : T_, nlo, nhi, ndst);                        \
    mem_fence_compiler();                                                                       \
  }
        MLA_PV_STEP(0) MLA_PV_STEP(1) MLA_PV_STEP(2) MLA_PV_STEP(3) MLA_PV_STEP(4)
        MLA_PV_STEP(5) MLA_PV_STEP(6) MLA_PV_STEP(7) MLA_PV_STEP(8) MLA_PV_STEP(9)
        MLA_PV_STEP(10) MLA_PV_STEP(11) MLA_PV_STEP(12) MLA_PV_STEP(13) MLA_PV_STEP(14)
        MLA_PV_STEP(15) MLA_PV_STEP(16) MLA_PV_STEP(17) MLA_PV_STEP(18) MLA_PV_STEP(19)
        MLA_PV_STEP(20) MLA_PV_STEP(21) MLA_PV_STEP(22) MLA_PV_STEP(23) MLA_PV_STEP(24)
        MLA_PV_STEP(25) MLA_PV_STEP(26) MLA_PV_STEP(27) MLA_PV_STEP(28) MLA_PV_STEP(29)
        MLA_PV_STEP(30) MLA_PV_STEP(31) MLA_PV_STEP(32) MLA_PV_STEP(33) MLA_PV_STEP(34)
        MLA_PV_STEP(35) MLA_PV_STEP(36) MLA_PV_STEP(37) MLA_PV_STEP(38) MLA_PV_STEP(39)
        MLA_PV_STEP(40) MLA_PV_STEP(41) MLA_PV_STEP(42) MLA_PV_STEP(43) MLA_PV_STEP(44)
        MLA_PV_STEP(45) MLA_PV_STEP(46) MLA_PV_STEP(47) MLA_PV_STEP(48) MLA_PV_STEP(49)
        MLA_PV_STEP(50) MLA_PV_STEP(51) MLA_PV_STEP(52) MLA_PV_STEP(53) MLA_PV_STEP(54)
        MLA_PV_STEP(55) MLA_PV_STEP(56) MLA_PV_STEP(57) MLA_PV_STEP(58) MLA_PV_STEP(59)
        MLA_PV_STEP(60) MLA_PV_STEP(61) MLA_PV_STEP(62) MLA_PV_STEP(63)
#undef MLA_PV_STEP
      }
      // the last step's copies (of nothing new) land before any buffer is
      // reused, and every wave is done with the last page
      wait_vm<0>();
      barrier();
      return over;
    };

    // page p0 into buffer 0, unless it went there before the epilogue of
    // the sequence ahead; then the queries
    if (!page_issued) {
      i32x4 lo, hi;
      page_rsrc_of(p0, pg_a, true, lo, hi);
      MLA_DMA_ALL(lo, hi, lds0);
    }
    load_q();
    // every wave runs the same passes: the page buffers and barriers are shared
    if (block_or<R128_WAVES>(run_pass(pass_tag<PASS_FIRST_REF>{}), lds_p, wave)) {
      run_pass(pass_tag<PASS_MAX_ONLY>{});
      run_pass(pass_tag<PASS_PRESET_REF>{});
    }

    // Every wave is past the last page and the flag words: both page
    // buffers are free. The next sequence's first page goes into buffer 0
    // now, so that its latency overlaps this sequence's epilogue, which
    // stages its rows in buffer 1.
    if (b < be) {
      int nL, npg_a;  // the next sequence's length and first page
      sload_2(seqlens + b + 1, uniform_ptr(a.block_table + (size_t)(b + 1) * a.bt_stride), nL,
              npg_a);
      const int nnpg = sched::seq_pages(nL);
      const int np1 = min(b + 1 == be ? p_end : nnpg, nnpg);
      if (np1 > 0) {  // pages 0 .. np1 - 1 of the next sequence are this worker's
        i32x4 lo, hi;
        make_rsrc(npg_a, min(64, nL) * 1152, lo, hi);
        MLA_DMA_ALL(lo, hi, lds0);
        next_page = true;
      }
    }

    // ---- epilogue. Lane l holds output columns 32tt + 8q + 4hf .. +3 of
    // row n, so direct stores would write 32 rows x 32 bytes each. O leaves
    // through LDS instead: a wave stages 128 columns of its 32 rows at a
    // time (scaled by 1 / lw) in its own quarter of the page buffers, free
    // once the passes are done, and reads them back two whole rows of 512
    // bytes per instruction, so every store writes full lines.
    {
      float lr = l, lwr = lw;
      {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(lr), __float_as_uint(lr),
                                                        false, false);
        lr = __uint_as_float(p[0]) + __uint_as_float(p[1]);
        const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(lwr),
                                                        __float_as_uint(lwr), false, false);
        lwr = __uint_as_float(q[0]) + __uint_as_float(q[1]);
      }
      float sc_o = lwr > 0.f ? 1.f / lwr : 0.f;
      const float lse_v = lr > 0.f ? (m + __log2f(lr)) * LN2 : -INFINITY;
      // the scale is laundered so that the products are formed tile by tile
      // rather than all 256 at once
      asm volatile("" : "+v"(sc_o));
      const bool to_part = nslots != 0;
      const size_t slot = (size_t)(s0 + split);
      constexpr int PITCH = 528;  // staged row: 128 fp32 + 16 bytes of bank skew
      static_assert(R128_WAVES * 32 * PITCH <= LY::TILE, "staging fits one page buffer");
      lds_char* const stage = lds_p + LY::TILE + wave * (32 * PITCH);
      const int row0 = rb * 128 + wave * 32;  // the wave's first row
      // the row bases stay global pointers: generic ones would make the
      // stores FLAT, which also count against the LDS counter, so every
      // staging read would wait for the stores before it
      __attribute__((address_space(1))) float* const part_base =
          (__attribute__((address_space(1))) float*)(a.part_o + (slot * TH + row0) * LY::DV);
      __attribute__((address_space(1))) uint16_t* const out_base =
          (__attribute__((address_space(1))) uint16_t*)(a.out + ((size_t)b * TH + row0) * LY::DV);
      auto staged = [&](auto part_tag) {
        constexpr bool PART = decltype(part_tag)::value;
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
          // Lane offsets are formed again from the lane index in every
          // chunk: kept from before the page loop they would be spilled
          // registers, and a reload waits for every store issued before it
          // (the memory counter retires in order).
          int lid = (int)threadIdx.x;
          asm volatile("" : "+v"(lid));
          const int ln = lid & 31, lh = (lid >> 5) & 1;
          // staging: lane (n, hf) writes row n; read-back: lane (cc, rr)
          // reads 16 bytes cc of row 2i + rr
          const uint32_t wr = (uint32_t)(ln * PITCH + 16 * lh);
          const uint32_t rd = (uint32_t)(lh * PITCH + 16 * ln);
          const uint32_t el = (uint32_t)(lh * LY::DV + 4 * ln + 128 * ch);
#pragma unroll
          for (int t4 = 0; t4 < 4; ++t4) {
            const int tt = 4 * ch + t4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x4 z = {o[tt][4 * q] * sc_o, o[tt][4 * q + 1] * sc_o,
                               o[tt][4 * q + 2] * sc_o, o[tt][4 * q + 3] * sc_o};
              *(__attribute__((address_space(3))) f32x4*)(stage + wr + 4 * (32 * t4 + 8 * q)) = z;
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          // a wave's LDS accesses run in issue order: the reads see the
          // writes. All sixteen reads go out before the first store, so
          // their latencies overlap (the query registers are free here);
          // read one at a time, each store waited for its own round trip.
          f32x4 v[16];
#pragma unroll
          for (int i = 0; i < 16; ++i)
            v[i] = *(const __attribute__((address_space(3))) f32x4*)(stage + rd + 2 * i * PITCH);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if constexpr (PART) {
              *(__attribute__((address_space(1))) f32x4*)(part_base + el + 2 * i * LY::DV) = v[i];
            } else {
              const u32x2 z = {pack_bf16x2(v[i][0], v[i][1]), pack_bf16x2(v[i][2], v[i][3])};
              *(__attribute__((address_space(1))) u32x2*)(out_base + el + 2 * i * LY::DV) = z;
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // A wave whose 32 rows run past T * H (only when T * H is not a
      // multiple of 32) stores straight from the accumulators, each lane
      // its own row if that row exists.
      auto direct = [&](auto part_tag) {
        constexpr bool PART = decltype(part_tag)::value;
        if (!row_ok) return;
#pragma unroll
        for (int tt = 0; tt < R128_NT; ++tt) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 z = {o[tt][4 * q] * sc_o, o[tt][4 * q + 1] * sc_o,
                             o[tt][4 * q + 2] * sc_o, o[tt][4 * q + 3] * sc_o};
            const uint32_t el = (uint32_t)(n * LY::DV + 32 * tt + 8 * q + 4 * hf);
            if constexpr (PART) {
              *(__attribute__((address_space(1))) f32x4*)(part_base + el) = z;
            } else {
              *(__attribute__((address_space(1))) u32x2*)(out_base + el) =
                  u32x2{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])};
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      const bool full = row0 + 32 <= TH;
      if (to_part) {
        if (full) staged(std::true_type{});
        else direct(std::true_type{});
      } else {
        if (full) staged(std::false_type{});
        else direct(std::false_type{});
      }
      if (row_ok && hf == 0) {
        if (to_part)
          a.part_lse[slot * TH + rho] = lse_v;
        else
          a.lse[(size_t)b * TH + rho] = lse_v;
      }
    }
    // No barrier here: the staging buffer (buffer 1) takes page copies again
    // only after the next sequence's first barrier, which every wave reaches
    // once its staged rows are stored; the next first page lands in buffer 0.
  }
}

#undef MLA_DMA_ALL
#undef MLA_DMA_ONE

hipError_t launch_decode128_kernel(const DecodeArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL(decode128_kernel, dim3(grid), dim3(64 * R128_WAVES), 0, st, a);
  return hipGetLastError();
}

}  // namespace mla
