// Fused paged attention decode for gfx950: one kernel walks a worker's
// pages, and per 64-token page computes scores on MFMA, masks them, updates
// the online softmax and accumulates P V on MFMA, writing only the final
// (or split-partial) result.
//
// Method: FlashAttention (KO) — tiling ("타일링 및 블록 처리"), the online
// softmax with a running max and running exp-sum ("온라인 Softmax 계산"), and
// one fused kernel for QK^T, masking, softmax and the product with V
// ("단일 CUDA 커널로의 연산 융합"). Paging: PagedAttention's block table
// (cited in "참고 문헌") with 64-token pages (FlashMLA blog, "기술 기반").
// Shapes: the MQA-absorb and GQA decode paths of the GQLA review ("1. Key
// Terms & Definitions").
//
// Work layout (gfx950, wave64, four compute waves per workgroup, plus four
// copy waves for the latent cache at 64 rows per workgroup):
//   * A workgroup owns one worker's range of pages (schedule.h) for one KV
//     head g and a block of 16*R query rows that share that head. Wave w
//     owns 16 rows (row group w % R); the KS = 4 / R waves of a row group
//     split every page's 64 keys into KS parts and keep separate softmax
//     states, merged through LDS when the worker's range of a sequence ends.
//   * Pages stream HBM -> LDS with global_load_lds_dwordx4 (no staging
//     registers), double-buffered: the next page is in flight while the
//     current one is computed. FP8 pages at 64 rows per workgroup instead
//     pass through the copy waves' registers, which dequantise them into
//     the bf16 latent layout.
//   * Scores are computed transposed, S^T[key][row] = K . Q^T, on 16x16x32
//     bf16 MFMA: lane l holds query row l % 16 and four keys per 16-key
//     block, so the row max and sum are in-lane reductions plus two
//     exchanges across the four 16-lane groups.
//   * Those registers, rounded to bf16, are directly the B operand of
//     O^T[dv][row] += V^T . P^T: an MFMA sums over its K slots in any order
//     as long as both operands agree, so the key in slot i of lane l is the
//     key that lane's score register already holds. The V^T operand is read
//     from the same LDS page with ds_read_b64_tr_b16 (4 consecutive keys of
//     one column per lane); for the latent cache V is columns 0..511 of the
//     K rows already in LDS, so every cache byte crosses HBM once.
//   * Q (72 registers) stays in registers for the whole sequence; O^T (128
//     fp32 registers for 512 columns) accumulates in registers.
#include "decode_device.h"
#include "schedule.h"

namespace mla {

template <int R, int KIND>
__global__ __launch_bounds__(64 * decode_waves(R, KIND)) void decode_kernel(DecodeArgs a) {
  // FP8 pages at 64 rows per workgroup: the copy waves dequantise every page
  // into the bf16 latent layout (each code times its token's power-of-two
  // scale, exact), so the compute waves run the bf16 path unchanged
  constexpr bool DEQ = KIND == KIND_MLA_FP8 && R == 4;
  using LY = Layout<DEQ ? KIND_MLA : KIND>;
  constexpr bool GQA = KIND != KIND_MLA && !DEQ;
  constexpr int NW = 4;           // compute waves
  // With copy waves, waves NW .. 2NW-1 issue every page copy and compute
  // nothing, so the compute waves never stall behind the address unit.
  constexpr bool PROD = decode_waves(R, KIND) > NW;
  constexpr int NWT = decode_waves(R, KIND);
  static_assert(!PROD || (R == 4 && !LY::FP8 && !GQA), "copy waves: latent bf16, 64 rows");
  // LDS operand prefetch distance; two waves per SIMD leave 256 registers a
  // wave, which hold O (128), Q (72) and two steps of operands (also the
  // fastest distance measured for this kernel: 2 < 1 < 3, 4, 6)
  constexpr int PFD = PROD ? 2 : PF;
  constexpr int KS = NW / R;      // waves sharing a row group (key split)
  // FP8 pages are half the size: with one row group, a loop step takes two
  // consecutive pages (a 128-key tile), so that each wave owns 32 keys of
  // one page and the per-step barriers and softmax cover twice the keys.
  constexpr int PPT = (LY::FP8 && R == 1) ? 2 : 1;  // pages per loop step
  constexpr int KW = 64 * PPT / KS;  // keys per wave per step
  constexpr int KB = KW / 16;        // 16-key score blocks per wave per step
  static_assert(!LY::FP8 || KW >= 32, "FP8 waves own at least 32 keys");
  constexpr int D = LY::D, DV = LY::DV;
  constexpr int KC = D / 32;      // MFMA K steps of the score product
  constexpr int NCB = DV / 16;    // 16-wide column blocks of the output
  constexpr int ROWS = 16 * R;
  constexpr int NDMA = PPT * LY::DMA_PER_TILE / NW;  // per wave per step
  static_assert(LY::DMA_PER_TILE % NW == 0 && NDMA < 64, "page copies split evenly");

  // the page buffers, reused at the end of a range for the key-part merge
  constexpr int MERGE_BYTES = (KS - 1) * R * (NCB * 4 + 3) * 64 * 4;
  constexpr int NB = PPT == 2 ? 2 : LY::NBUF;  // buffers of PPT pages each
  constexpr int STEP_BYTES = PPT * LY::TILE;
  constexpr int LDS_BYTES = NB * STEP_BYTES > MERGE_BYTES ? NB * STEP_BYTES : MERGE_BYTES;
  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];
  lds_char* const lds_p = LDS_PTR(char, lds);
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds_p;

  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6);
  const bool producer = PROD && wave >= NW;
  const int cw = PROD ? wave - NW : wave;  // index among the copying waves
  const int lane = tid & 63;
  const int n = lane & 15;     // query row within the wave's 16
  const int g4 = lane >> 4;    // 16-lane group
  const int rg = wave % R;     // row group
  const int ks = wave / R;     // key part

  int w, rb;
  decode_block_id(blockIdx.x, a.W, a.G * a.nrb, w, rb);
  const int g = rb / a.nrb;
  const int rblk = rb - g * a.nrb;

  // a plan made for another geometry: leave every output untouched rather
  // than index records or slots that belong to a different layout
  // (bitwise, not short-circuit: the six words load in one round trip)
  const int32_t* hdr = a.meta;
  const int32_t h_magic = hdr[sched::H_MAGIC], h_w = hdr[sched::H_W], h_b = hdr[sched::H_B],
                h_rows = hdr[sched::H_ROWS], h_g = hdr[sched::H_G], h_dv = hdr[sched::H_DV];
  if ((h_magic != sched::PLAN_MAGIC) | (h_w != a.W) | (h_b != a.B) | (h_rows != a.T * a.H) |
      (h_g != a.G) | (h_dv != LY::DV))
    return;
  const int32_t* rec = sched::records(a.meta) + w * sched::REC;
  const int bs = uniform(rec[sched::R_B_START]);
  const int be = uniform(rec[sched::R_B_END]);
  if (be < bs) return;

  const int hpg = a.H / a.G;
  const int r = rblk * ROWS + rg * 16 + n;  // row within this KV head
  const bool row_ok = !producer && r < a.M;
  const int t = row_ok ? r / hpg : 0;
  const int h = g * hpg + (row_ok ? r - t * hpg : 0);
  const int rho = t * a.H + h;               // output row within a sequence
  const int TH = a.T * a.H;

  // ---- per-lane LDS offsets (bytes, relative to a page buffer) ----
  // Score operand: key ks*KW + 16kb + n, K step c covers columns 32c .. 32c+31,
  // of which this lane reads chunk 4c + g4. With an XOR below 8 the 8-chunk
  // group stays put, so two offsets (c even / odd) plus 128 (c >> 1) cover
  // every step, rope included; the 4-bit XOR reaches across the group, so
  // each step has its own offset.
  constexpr int NQO = LY::K_XOR8 ? 2 : 4;
  const int xn = LY::k_xor(n);
  uint32_t qk_off[NQO];
#pragma unroll
  for (int q = 0; q < NQO; ++q)
    qk_off[q] = (ks * KW + n) * LY::K_PITCH + 16 * ((4 * q + g4) ^ xn);
  // V^T operand by transposed reads: 16-lane group g4 reads keys
  // 4*g4 + (j>>2) (+ a multiple of 16) at columns 16cb + 4(j&3) .. +3, i.e.
  // chunk 2cb + (j&3)/2; with an XOR below 8, 4 offsets (cb & 3) plus 128
  // (cb >> 2), else one per column block.
  constexpr int NVO = LY::V_XOR8 ? 4 : 8;
  const int j16 = lane & 15;
  const int vkey = 4 * g4 + (j16 >> 2);
  const int xv = LY::v_xor(vkey);
  uint32_t v_off[NVO];
#pragma unroll
  for (int q = 0; q < NVO; ++q)
    v_off[q] = LY::V_BASE + (ks * KW + vkey) * LY::V_PITCH +
               16 * ((2 * q + ((j16 & 3) >> 1)) ^ xv) + 8 * (j16 & 1);

  // FP8 pages. The score read of block kb takes row krow(kb, n) of the
  // wave's keys, 8 codes (columns 32c + 8g4 ..); the rows of the blocks are
  // chosen so that score register i of lane group g4 in blocks 2c and 2c+1
  // holds the key that the transposed V read (ds_read_b64_tr_b8: lane j of
  // group g4 gets rows 8g4 .. 8g4+7 of column j) puts in MFMA slot i:
  // krow(kb, a) = 32(kb/2) + 8(a/4) + 4(kb%2) + a%4 covers each 32 keys with
  // two blocks.
  auto krow = [](int kb, int a_) {
    return 32 * (kb >> 1) + 8 * (a_ >> 2) + 4 * (kb & 1) + (a_ & 3);
  };
  constexpr int KB8 = LY::FP8 ? KB : 1;
  uint32_t k8_off[KB8][2], sc_off[KB8], v8_off[4];
  if constexpr (LY::FP8) {
    // this wave's keys lie in page slot ps of the step, from row r0 on
    const uint32_t ps = (uint32_t)((ks * KW) >> 6) * LY::TILE;
    const int r0 = (ks * KW) & 63;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int row = r0 + krow(kb, n);
      const int y = LY::k_xor(row);
#pragma unroll
      for (int cp = 0; cp < 2; ++cp)
        k8_off[kb][cp] = ps + row * LY::K_PITCH + 16 * ((2 * cp + (g4 >> 1)) ^ y) + 8 * (g4 & 1);
      sc_off[kb] = ps + LY::SCALE_OFF + 4 * (r0 + krow(kb, 4 * g4));
    }
    const int vrow = r0 + 8 * g4 + (j16 >> 1);
    const int yv = LY::v_xor(vrow);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v8_off[q] = ps + vrow * LY::V_PITCH + 16 * (q ^ yv) + 8 * (j16 & 1);
  }

  // The sequences of the worker's range. With copy waves the two roles run
  // separate instances of this loop (CW: a copy wave), meeting at the same
  // barriers, so that neither keeps the other's registers live.
  auto seq_loop = [&](auto copy_role) {
  constexpr bool CW = decltype(copy_role)::value;
  for (int b = bs; b <= be; ++b) {
    const int L = uniform(a.seqlens[b]);
    const int npg = sched::seq_pages(L);
    int p0, p1;
    sched::page_range(rec, b, bs, be, npg, &p0, &p1);
    p0 = uniform(p0);
    p1 = uniform(p1);
    const int s0 = uniform(a.slots[b]);
    const int nslots = uniform(a.slots[b + 1]) - s0;

    if (npg == 0) {
      if (!CW && (b > bs || rec[sched::R_OWNS_FIRST]) && row_ok && ks == 0) {
        uint16_t* o = a.out + ((size_t)b * TH + rho) * DV;
        for (int cb = 0; cb < NCB; ++cb) *(u32x2*)(o + 16 * cb + 4 * g4) = u32x2{0u, 0u};
        if (g4 == 0) a.lse[(size_t)b * TH + rho] = -INFINITY;
      }
      continue;
    }
    if (p0 >= p1) continue;
    const int split = b == bs ? rec[sched::R_SPLIT0] : 0;
    const int32_t* bt = a.block_table + (size_t)b * a.bt_stride;

    // FP8 pages through the copy waves' registers: 16-byte unit u = 64i +
    // lane (i = cw + NW t) holds codes 16x .. 16x + 15 of row r = u / 36,
    // x = u % 36, which become bf16 chunks 2x and 2x + 1 of LDS row r; rows
    // past the sequence end repeat its last row, scale included
    constexpr int DQ_T = DEQ ? 36 / NW : 1;
    auto load_codes = [&](int j, u32x4 (&dq)[DQ_T], float& scale) {
      const int page = sload(uniform_ptr(bt + j));
      const int nv = uniform(min(64, L - 64 * j));
      const char* pbase = uniform_ptr((const char*)a.k + (size_t)page * (64 * 576));
#pragma unroll
      for (int t = 0; t < DQ_T; ++t) {
        const int u = 64 * (cw + NW * t) + lane;
        const int r = u / 36, x = u - 36 * r;
        dq[t] = __builtin_nontemporal_load((const u32x4*)(pbase + min(r, nv - 1) * 576 + 16 * x));
      }
      scale = a.kscale[(size_t)page * 64 + min(lane, nv - 1)];
    };
    auto store_page = [&](const u32x4 (&dq)[DQ_T], float scale, int buf) {
      lds_char* const dst = lds_p + buf * STEP_BYTES;
#pragma unroll
      for (int t = 0; t < DQ_T; ++t) {
        const int u = 64 * (cw + NW * t) + lane;
        const int r = u / 36, x = u - 36 * r;
        const float sc = __shfl(scale, r);  // lane r holds row r's scale
        u32x4 c0, c1;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          c0[2 * k] = fp8x2_bf16x2_scaled<false>(dq[t][k], sc);
          c0[2 * k + 1] = fp8x2_bf16x2_scaled<true>(dq[t][k], sc);
          c1[2 * k] = fp8x2_bf16x2_scaled<false>(dq[t][k + 2], sc);
          c1[2 * k + 1] = fp8x2_bf16x2_scaled<true>(dq[t][k + 2], sc);
        }
        const int y = r & 7;
        typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
        *(lds_u32x4*)(dst + r * LY::K_PITCH + 16 * ((2 * x) ^ y)) = c0;
        *(lds_u32x4*)(dst + r * LY::K_PITCH + 16 * ((2 * x + 1) ^ y)) = c1;
      }
    };

    // copy page j of sequence b to LDS byte dst
    auto issue_page = [&](int j, uint32_t dst) {
      const int page = sload(uniform_ptr(bt + j));
      const int nv = uniform(min(64, L - 64 * j));
      if constexpr (LY::FP8) {
        // codes: a contiguous 36 KiB block, copied like the latent page; then
        // every wave copies the page's 64 scales to the same LDS words (the
        // same bytes, so the waves need not agree on who does it)
        const char* pbase = uniform_ptr((const char*)a.k + (size_t)page * LY::SCALE_OFF);
#pragma unroll
        for (int t = 0; t < 36 / NW; ++t) {
          const int i = cw + NW * t;
          const int u = 64 * i + lane;
          const int r = u / 36, x = u - 36 * r;
          dma16(dst + 1024 * i, pbase, min(r, nv - 1) * LY::K_PITCH + 16 * (x ^ LY::k_xor(r)));
        }
        const char* sbase = uniform_ptr((const char*)a.kscale + (size_t)page * 256);
        dma4(dst + LY::SCALE_OFF, sbase, 4 * min(lane, nv - 1));
      } else if constexpr (!GQA) {
        // the page is one contiguous 72 KiB block in HBM and in LDS: copy i
        // fills LDS bytes 1024i .. 1024i+1023, 16-byte unit u = 64i + lane,
        // i.e. chunk x of row r; rows past the sequence end repeat its last
        // row (finite data that the mask gives weight 0)
        const char* pbase = uniform_ptr((const char*)a.k + (size_t)page * LY::TILE);
#pragma unroll
        for (int t = 0; t < LY::DMA_PER_TILE / NW; ++t) {
          const int i = cw + NW * t;
          const int u = 64 * i + lane;
          const int r = u / 72, x = u - 72 * r;
          const uint32_t vo = min(r, nv - 1) * LY::K_PITCH + 16 * (x ^ LY::k_xor(r));
          dma16(dst + 1024 * i, pbase, vo);
        }
      } else {
        // KV head g's rows of the page: K rows of KC16 chunks, V rows of VC16
        // chunks, tokens G heads apart in HBM; copy i of K (or V) holds
        // 16-byte units u = 64i + lane, chunk x of row r, as above
        constexpr int KC16 = LY::D / 8, VC16 = LY::DV / 8;
        static_assert(KC16 % NW == 0 && VC16 % NW == 0, "copies split evenly");
        const uint32_t kstride = (uint32_t)a.G * (LY::D * 2);  // bytes between tokens
        const uint32_t vstride = (uint32_t)a.G * (LY::DV * 2);
        const size_t row0 = (size_t)page * 64 * a.G + g;
        const char* kbase = uniform_ptr((const char*)a.k + row0 * (LY::D * 2));
        const char* vbase = uniform_ptr((const char*)a.v + row0 * (LY::DV * 2));
#pragma unroll
        for (int t = 0; t < KC16 / NW; ++t) {
          const int i = cw + NW * t;
          const int u = 64 * i + lane;
          const int r = u / KC16, x = u - KC16 * r;
          dma16(dst + 1024 * i, kbase, min(r, nv - 1) * kstride + 16 * (x ^ LY::k_xor(r)));
        }
#pragma unroll
        for (int t = 0; t < VC16 / NW; ++t) {
          const int i = cw + NW * t;
          const int u = 64 * i + lane;
          const int r = u / VC16, x = u - VC16 * r;
          dma16(dst + LY::V_BASE + 1024 * i, vbase,
                min(r, nv - 1) * vstride + 16 * (x ^ LY::v_xor(r)));
        }
      }
    };

    // queries of this lane's row, as B operands of the score MFMA
    bf16x8 qf[KC];
    if constexpr (!CW) {
      const uint16_t* qrow = a.q + ((size_t)b * TH + rho) * D;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        u32x4 x = row_ok ? *(const u32x4*)(qrow + 32 * c + 8 * g4) : u32x4{0u, 0u, 0u, 0u};
        qf[c] = __builtin_bit_cast(bf16x8, x);
      }
      // The page copies are inline asm the compiler does not count; consume
      // q here so that its own wait for these loads sits before the page
      // loop and not inside it.
#pragma unroll
      for (int c = 0; c < KC; ++c) asm volatile("" ::"v"(qf[c]));
    }
    const int vis = a.causal ? min(L - a.T + 1 + t, L) : L;

    // One pass over the page range, accumulating O, l and the row reference
    // m. FIXED: a row's m is the max of the first page on which the row sees
    // a key (O and l are still exactly 0 then) and never moves afterwards;
    // weights exp2(s - m) only grow, and fp32 holds them exactly in relative
    // terms, so the pass is exact unless a later page exceeds m by more than
    // REF_LIMIT, which it reports. Otherwise: the lazily rescaled online
    // softmax, which cannot overflow. The fixed pass touches O with MFMA
    // only, so O stays in the accumulator registers.
    // l sums the weights as computed (for the LSE); lw sums them as the P V
    // MFMA receives them, rounded to bf16, and normalises the output, whose
    // weights then form an exact convex combination (with FP8 the weights
    // carry power-of-two token scales, which commute with the rounding)
    f32x4 o[NCB];
    float m, l, lw;
    auto run_range = [&](auto fixed_tag) -> bool {
    constexpr bool FIXED = decltype(fixed_tag)::value;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    l = 0.f;
    lw = 0.f;
    bool over = false;

    // a step's PPT pages from page j into buffer buf; past the worker's
    // range the slot gets page j again (finite data whose keys are masked),
    // so every wave issues the same number of copies per step
    auto issue_step = [&](int j, int buf) {
#pragma unroll
      for (int pp = 0; pp < PPT; ++pp)
        issue_page(j + pp < p1 ? j + pp : j, lds0 + buf * STEP_BYTES + pp * LY::TILE);
    };
    // step j's scores, softmax update and P V from step buffer cur
    auto compute_step = [&](int j, int cur) {
      // LDS operands are addressed as a per-lane pointer into this page's
      // buffer plus a compile-time byte offset, which the compiler folds
      // into the offset field of the LDS read.
      lds_char* const buf = lds_p + cur * STEP_BYTES;
      const lds_char* kp[NQO];
#pragma unroll
      for (int q = 0; q < NQO; ++q) kp[q] = buf + qk_off[q];
      const lds_char* vp[NVO];
#pragma unroll
      for (int q = 0; q < NVO; ++q) vp[q] = buf + v_off[q];
      const lds_char* kp8[KB8][2];
      const lds_char* vp8[4];
      if constexpr (LY::FP8) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          kp8[kb][0] = buf + k8_off[kb][0];
          kp8[kb][1] = buf + k8_off[kb][1];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) vp8[q] = buf + v8_off[q];
      }

      // S^T = K . Q^T, one 16-key block per kb. Steps run d-chunk-major
      // (st = c * KB + kb) into four accumulators (st % 4), so consecutive
      // MFMAs never depend on each other; blocks that own several
      // accumulators sum them afterwards. K fragments are read PFD steps
      // ahead of the MFMA that uses them.
      auto k_frag = [&](int st) -> bf16x8 {
        const int c = st / KB, kb = st % KB;
        if constexpr (LY::FP8) {
          const lds_char* p = kp8[kb][c & 1] + 64 * (c >> 1);
          const u32x2 w = *(const __attribute__((address_space(3))) u32x2*)p;
          return fp8x8_bf16x8(w[0], w[1]);
        }
        const lds_char* p = LY::K_XOR8 ? kp[c & 1] + kb * 16 * LY::K_PITCH + 128 * (c >> 1)
                                       : kp[c % NQO] + kb * 16 * LY::K_PITCH;
        return *(const __attribute__((address_space(3))) bf16x8*)p;
      };
      constexpr int NQK = KB * KC;
      constexpr int PFK = NQK < PFD ? NQK : PFD;
      static_assert(KB <= 4 && 4 % KB == 0, "score blocks map onto four accumulators");
      f32x4 acc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      bf16x8 kf[PFK + 1];
#pragma unroll
      for (int st = 0; st < PFK; ++st) kf[st] = k_frag(st);
#pragma unroll
      for (int st = 0; st < NQK; ++st) {
        if (st + PFK < NQK) kf[(st + PFK) % (PFK + 1)] = k_frag(st + PFK);
        acc[st % 4] = mfma16(kf[st % (PFK + 1)], qf[st / KB], acc[st % 4]);
        mem_fence_compiler();
      }
      f32x4 s[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        s[kb] = acc[kb];
#pragma unroll
        for (int i = kb + KB; i < 4; i += KB) s[kb] += acc[i];
      }

      // scale, mask, running max over this wave's keys (FP8: times each
      // key's token scale, which multiplies the whole K row)
      float tmax = -INFINITY;
      const int kbase = 64 * j + ks * KW;
      // a wave's keys lie in one page, which must be inside the worker's range
      const bool page_ok = PPT == 1 || j + ((ks * KW) >> 6) < p1;
      f32x4 ksc[KB8];
      if constexpr (LY::FP8) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          ksc[kb] = *(const __attribute__((address_space(3))) f32x4*)(buf + sc_off[kb]);
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kbase + (LY::FP8 ? krow(kb, 4 * g4) : 16 * kb + 4 * g4) + i;
          const float sc = LY::FP8 ? a.scale_log2 * ksc[kb][i] : a.scale_log2;
          const float x = (page_ok && key < vis) ? s[kb][i] * sc : -INFINITY;
          s[kb][i] = x;
          tmax = fmaxf(tmax, x);
        }
      tmax = max4groups(tmax);
      if constexpr (FIXED) {
        if (m == -INFINITY) m = tmax;
        over = over || tmax > m + REF_LIMIT;
      } else {
        // Lazy rescale: m is a per-row reference, not the exact running
        // max. Weights are exp2(s - m) <= 2^RESCALE_SLACK; only when a page
        // raises a row's max by more than that (or gives the row its first
        // key) are l and O rescaled to the new reference. l and O always
        // share the same reference, so O / l and m + log2(l) are exact.
        const bool need = tmax > m + RESCALE_SLACK;
        if (__any(need)) {
          // rows that do not need it keep alpha = 1 (a row that has seen no
          // key yet has m = -inf, and exp2(m - m) would be NaN)
          const float alpha = need ? fast_exp2(m - tmax) : 1.f;  // 0 when m = -inf
          l *= alpha;
          lw *= alpha;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) o[cb] *= alpha;
          m = need ? tmax : m;
        }
      }
      const float m_use = m == -INFINITY ? 0.f : m;
      float psum = 0.f, wsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fast_exp2(s[kb][i] - m_use);
          // FP8: the V row is scaled by its token scale too; l is not
          s[kb][i] = LY::FP8 ? p * ksc[kb][i] : p;
          psum += p;
          wsum += (float)(__bf16)p;
        }
      l += sum4groups(psum);
      lw += sum4groups(wsum);

      // O^T += V^T . P^T
      if constexpr (KW >= 32) {
        // K step c covers this wave's keys 32c .. 32c+31; slot i of lane l
        // holds key 32c + 16(i/4) + 4(l/16) + i%4 = score block 2c + i/4,
        // register i%4.
        constexpr int PC = KW / 32;
        bf16x8 pf[PC];
#pragma unroll
        for (int c = 0; c < PC; ++c) {
          u32x4 x;
          x[0] = pack_bf16x2(s[2 * c][0], s[2 * c][1]);
          x[1] = pack_bf16x2(s[2 * c][2], s[2 * c][3]);
          x[2] = pack_bf16x2(s[2 * c + 1][0], s[2 * c + 1][1]);
          x[3] = pack_bf16x2(s[2 * c + 1][2], s[2 * c + 1][3]);
          pf[c] = __builtin_bit_cast(bf16x8, x);
        }
        // steps run key-chunk-major (st = c * NCB + cb): consecutive MFMAs
        // hit different output blocks; V^T fragments are read PFD steps ahead
        auto v_frag = [&](int st) -> bf16x8 {
          const int c = st / NCB, cb = st % NCB;
          if constexpr (LY::FP8) {
            const lds_char* p = vp8[cb & 3] + 64 * (cb >> 2) + (32 * c) * LY::V_PITCH;
            const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p);
            return fp8x8_bf16x8((uint32_t)w[0], (uint32_t)w[1]);
          }
          const lds_char* p = (32 * c) * LY::V_PITCH +
                              (LY::V_XOR8 ? vp[cb & 3] + 128 * (cb >> 2) : vp[cb % NVO]);
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
          const bf16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 16 * LY::V_PITCH));
          return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        constexpr int NST = NCB * PC;
        constexpr int PFV = NST < PFD ? NST : PFD;
        bf16x8 vf[PFV + 1];
#pragma unroll
        for (int st = 0; st < PFV; ++st) vf[st] = v_frag(st);
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          if (st + PFV < NST) vf[(st + PFV) % (PFV + 1)] = v_frag(st + PFV);
          o[st % NCB] = mfma16(vf[st % (PFV + 1)], pf[st / NCB], o[st % NCB]);
          mem_fence_compiler();
        }
      } else {
        // 16 keys per wave: 16x16x16 MFMA, slot i of lane l holds key
        // 4(l/16) + i, exactly score register i.
        u32x2 px;
        px[0] = pack_bf16x2(s[0][0], s[0][1]);
        px[1] = pack_bf16x2(s[0][2], s[0][3]);
        const bf16x4 pf = __builtin_bit_cast(bf16x4, px);
        auto v_frag = [&](int cb) -> bf16x4 {
          const lds_char* p = LY::V_XOR8 ? vp[cb & 3] + 128 * (cb >> 2) : vp[cb % NVO];
          return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
        };
        constexpr int PFV = NCB < PFD ? NCB : PFD;
        bf16x4 vf[PFV + 1];
#pragma unroll
        for (int cb = 0; cb < PFV; ++cb) vf[cb] = v_frag(cb);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          if (cb + PFV < NCB) vf[(cb + PFV) % (PFV + 1)] = v_frag(cb + PFV);
          o[cb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[cb % (PFV + 1)], pf, o[cb], 0, 0, 0);
          mem_fence_compiler();
        }
      }
    };

    if constexpr (PROD) {
      // The copy waves fill one buffer while the compute waves read the
      // other. At the barrier opening step j, step j's copies have landed
      // (each copy wave waited for its own) and step j - 1's compute is
      // done, so step j + 1 may refill that buffer.
      if constexpr (CW && DEQ) {
        // two pages in registers (sets A and B by page parity): step j
        // dequantises page j into buffer cur and sends out page j + 2's
        // loads into the set it frees; the barrier opens page j once this
        // wave's LDS writes are done
        u32x4 dqa[DQ_T], dqb[DQ_T];
        float sa = 0.f, sb = 0.f;
        if (p0 < p1) load_codes(p0, dqa, sa);
        if (p0 + 1 < p1) load_codes(p0 + 1, dqb, sb);
        int cur = 0;
        for (int j = p0; j < p1; j += 2) {
          store_page(dqa, sa, cur);
          if (j + 2 < p1) load_codes(j + 2, dqa, sa);
          wait_lgkm0();
          barrier();
          cur ^= 1;
          if (j + 1 < p1) {
            store_page(dqb, sb, cur);
            if (j + 3 < p1) load_codes(j + 3, dqb, sb);
            wait_lgkm0();
            barrier();
            cur ^= 1;
          }
        }
      } else if constexpr (CW) {
        if (p0 < p1) issue_step(p0, 0);
        int cur = 0;
        for (int j = p0; j < p1; ++j) {
          wait_vm<0>();
          barrier();
          if (j + 1 < p1) issue_step(j + 1, cur ^ 1);
          cur ^= 1;
        }
      } else {
        int cur = 0;
        for (int j = p0; j < p1; ++j) {
          barrier();
          compute_step(j, cur);
          cur ^= 1;
        }
      }
      barrier();  // the last buffer is read before anything refills it
    } else {
      // ring of NB step buffers: NB - 1 steps in flight ahead of the one
      // computed; step j + (NB - 1) PPT goes to the buffer step j - PPT used,
      // which every wave left at the barrier ending that step
#pragma unroll
      for (int k = 0; k < NB - 1; ++k)
        if (p0 + k * PPT < p1) issue_step(p0 + k * PPT, k);
      int cur = 0;
      for (int j = p0; j < p1; j += PPT) {
        if (j + (NB - 1) * PPT < p1) issue_step(j + (NB - 1) * PPT, cur == 0 ? NB - 1 : cur - 1);
        // this wave's copies still in flight after step j's: those of the
        // steps issued after it, at most NB - 1
        const int ahead = min(NB - 1, (p1 - 1 - j) / PPT);
        if constexpr (NB == 2) {
          if (ahead > 0) wait_vm<NDMA>(); else wait_vm<0>();
        } else {
          static_assert(NB == 4 && 3 * NDMA < 64, "wait counts fit vmcnt");
          if (ahead >= 3) wait_vm<3 * NDMA>();
          else if (ahead == 2) wait_vm<2 * NDMA>();
          else if (ahead == 1) wait_vm<NDMA>();
          else wait_vm<0>();
        }
        barrier();
        compute_step(j, cur);
        barrier();  // every wave is done with this buffer before it is refilled
        cur = cur + 1 == NB ? 0 : cur + 1;
      }
    }
    return over;
    };
    // every wave runs the same passes: the page buffers and barriers are shared
    if (block_or<NWT>(run_range(std::true_type{}), lds_p, wave)) run_range(std::false_type{});

    // merge the key parts of each row group through LDS (page buffers are
    // free: every copy has landed and every wave has passed the last barrier)
    if constexpr (KS > 1) {
      float* red = (float*)lds;  // [KS-1][R][NCB*4 + 3][64] floats
      constexpr int PER = NCB * 4 + 3;
      static_assert((KS - 1) * R * PER * 64 * 4 <= LDS_BYTES, "the merge fits in LDS");
      if (ks > 0) {
        float* my = red + ((ks - 1) * R + rg) * PER * 64 + lane;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) my[(cb * 4 + i) * 64] = o[cb][i];
        my[(NCB * 4) * 64] = m;
        my[(NCB * 4 + 1) * 64] = l;
        my[(NCB * 4 + 2) * 64] = lw;
      }
      __syncthreads();
      if (ks == 0) {
#pragma unroll
        for (int part = 1; part < KS; ++part) {
          const float* ot = red + ((part - 1) * R + rg) * PER * 64 + lane;
          const float m2 = ot[(NCB * 4) * 64], l2 = ot[(NCB * 4 + 1) * 64];
          const float mm = fmaxf(m, m2);
          const float mu = mm == -INFINITY ? 0.f : mm;
          const float a1 = fast_exp2(m - mu), a2 = fast_exp2(m2 - mu);
          l = a1 * l + a2 * l2;
          lw = a1 * lw + a2 * ot[(NCB * 4 + 2) * 64];
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[cb][i] = a1 * o[cb][i] + a2 * ot[(cb * 4 + i) * 64];
          m = mm;
        }
      }
      __syncthreads();  // the buffers are refilled by the next sequence
    }

    // epilogue: normalise; lane l holds dv = 16cb + 4(l/16) + i
    if (!CW && row_ok && ks == 0) {
    const float inv = lw > 0.f ? 1.f / lw : 0.f;
    const float lse_v = l > 0.f ? (m + __log2f(l)) * LN2 : -INFINITY;
    if (nslots == 0) {
      uint16_t* orow = a.out + ((size_t)b * TH + rho) * DV;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        u32x2 x;
        x[0] = pack_bf16x2(o[cb][0] * inv, o[cb][1] * inv);
        x[1] = pack_bf16x2(o[cb][2] * inv, o[cb][3] * inv);
        *(u32x2*)(orow + 16 * cb + 4 * g4) = x;
      }
      if (g4 == 0) a.lse[(size_t)b * TH + rho] = lse_v;
    } else {
      const size_t slot = (size_t)(s0 + split);
      float* prow = a.part_o + (slot * TH + rho) * DV;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) *(f32x4*)(prow + 16 * cb + 4 * g4) = o[cb] * inv;
      if (g4 == 0) a.part_lse[slot * TH + rho] = lse_v;
    }
    }
  }
  };
  if constexpr (PROD) {
    if (producer) seq_loop(std::true_type{});
    else seq_loop(std::false_type{});
  } else {
    seq_loop(std::false_type{});
  }
}

template <int R, int KIND>
static hipError_t launch_decode(const DecodeArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<R, KIND>), dim3(grid), dim3(64 * decode_waves(R, KIND)), 0,
                     st, a);
  return hipGetLastError();
}

template <int KIND>
static hipError_t launch_kind(const DecodeArgs& a, int row_groups, int grid, hipStream_t st) {
  switch (row_groups) {
    case 1: return launch_decode<1, KIND>(a, grid, st);
    case 2: return launch_decode<2, KIND>(a, grid, st);
    case 4: return launch_decode<4, KIND>(a, grid, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_kernel(const DecodeArgs& a, int row_groups, int kind, int grid,
                                hipStream_t st) {
  switch (kind) {
    case KIND_MLA: return launch_kind<KIND_MLA>(a, row_groups, grid, st);
    case KIND_GQA: return launch_kind<KIND_GQA>(a, row_groups, grid, st);
    case KIND_GQA_ROPE: return launch_kind<KIND_GQA_ROPE>(a, row_groups, grid, st);
    case KIND_MLA_FP8: return launch_kind<KIND_MLA_FP8>(a, row_groups, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace mla
