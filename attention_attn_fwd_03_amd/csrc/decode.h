// Paged split-KV decode on gfx950.
//
// One query token per sequence reads its KV cache through a block table of
// 16-token pages ("GPU Datapath: Where Every Byte Moves", section D). The
// cached context is cut into contiguous page-aligned groups; each group
// produces a normalised partial output and its log-sum-exp ("Why your local
// LLM feels dumber than it is", section "Why the calculation is split into
// groups"), merged afterwards by the combine kernel.
//
// Split plan: split s of a sequence covers pages [s P, (s+1) P) of it, with
// P = ceil(max_pages / num_splits) from the block-table width; a sequence
// shorter than the table leaves its trailing splits empty (merged as (0, -inf)).
// For one sequence that fills the table this is the contiguous equal-count
// partition of the pages.
//
// Work decomposition: one workgroup of 8 waves per (group of HW kv heads,
// sequence, split), HW = 8, 4, 2 or 1, with 8/HW waves per kv head taking the
// split's pages in turn. With HW = Hkv a workgroup reads every kv head of a
// page together, i.e. whole 16-token pages as contiguous runs of token rows,
// instead of one head's slice of each row. The G = Hq/Hkv query heads that
// share a kv head are served together, so each K/V byte is read from HBM once.
// Each wave keeps its own running max / sum / output; the waves of a kv head
// are merged through LDS in a fixed order at the end.
//
// Numerics variants (STUDY): the same kernel can store other split records
// and round at other points, so that the decode programs compared in "Why
// your local LLM feels dumber than it is" (section "Backend names expand into
// four decode algorithms") can be run on this kernel's own arithmetic:
//   record 0: normalised fp32 partial + LSE (the default above);
//   record 1: fp32 numerator + reference max + normaliser;
//   record 2: normalised partial rounded to bf16 + reference max + normaliser;
//   record 3: numerator rounded to bf16 + reference max + normaliser;
//   rounded_l: the normaliser sums the rounded weights that enter P.V
//              instead of the fp32 ones;
//   RR: tiles of 2^tile_shift pages dealt to the splits round robin (tile j
//       to split j mod S) instead of contiguous page ranges;
//   PF16: P rounded to fp16 instead of bf16, with V converted to fp16 (exact
//         for bf16 values inside fp16's normal range) for an fp16 P.V MFMA.
// The reference max is the running max the weights were taken against (in
// log2 units of the scaled score); merge kernels for records 1-3 are in
// combine.h.
//
// Per page (16 tokens) a wave computes S^T = K . Q^T with 16x16x32 bf16 MFMAs
// (rows: tokens, columns: query heads, padded to 16), so lane l holds query
// head l%16 for tokens 4(l/16)..4(l/16)+3. Those four probabilities, rounded
// to bf16, are directly the B operand of a 16x16x16 MFMA computing
// O^T += V^T . P^T; the V^T operand comes from the page staged in LDS and read
// back with the transposing ds_read_b64_tr_b16.
#pragma once
#include "balance.h"
#include "common.h"

namespace miattn {

struct DecodeArgs {
  const uint16_t* q;            // [B, Hq, D] bf16
  const uint16_t* k_cache;      // [num_pages, 16, Hkv, D] bf16
  const uint16_t* v_cache;
  const int32_t* block_table;   // [B, max_pages]
  const int32_t* seq_lens;      // [B]
  float* part_o;                // [B*Hq, S, D] fp32   (num_splits > 1)
  float* part_lse;              // [B*Hq, S] fp32
  float* part_m;                // [B*Hq, S] fp32 reference max, log2 units (records 1-3)
  float* part_l;                // [B*Hq, S] fp32 normaliser (records 1-3)
  uint16_t* o;                  // [B, Hq, D] bf16     (num_splits == 1)
  float* lse;                   // [B, Hq] fp32 or null
  int batch;
  int max_pages;
  int num_pages;
  int num_q_heads;
  int num_kv_heads;
  int group;                    // G = Hq / Hkv (<= 16: the columns of the score tile)
  int heads_per_wg;             // HW: kv heads served by one workgroup (8, 4, 2 or 1)
  int num_splits;
  float c;                      // scale * log2(e)
  int record;                   // STUDY: split record 0-3
  int rounded_l;                // STUDY: normaliser sums the rounded weights
  int tile_shift;               // RR: log2(pages per tile)
  int balance_units;            // > 0: length-proportional groups (balance.h), U per head group
  int32_t* plan_table;          // balanced: [2][batch] first group and group count per sequence
};

constexpr int kDecodeWaves = 8;
constexpr int kDecodeThreads = 64 * kDecodeWaves;
// query heads per kv head: the 16 columns of a wave's score tile (the merge
// area of 16 heads fits inside the page staging area at every head_dim)
constexpr int kDecodeMaxGroup = 16;
constexpr int kPage = 16;
// Lazy rescaling: the running max only moves when a page's max exceeds it by
// more than this many powers of two, so the stored probabilities stay <= 2^8.
constexpr float kRescaleThreshold = 8.0f;

template <int D>
struct DecodeSmem {
  static constexpr int kRowElems = D + 8;                         // padded K/V row (bf16)
  static constexpr int kStageBytes = kDecodeWaves * 2 * kPage * kRowElems * 2;   // K and V per wave
  static constexpr int kMergeBytes = kDecodeWaves * kDecodeMaxGroup * D * 4;
  static constexpr int kBytes = (kStageBytes > kMergeBytes ? kStageBytes : kMergeBytes)
                                + 2 * kDecodeWaves * 16 * 4;      // m and l per wave and head
};

__device__ __forceinline__ float round_bf16(float x) { return bf16lo_to_f32(pack_bf16x2(x, 0.f)); }

// PF = pages each wave keeps in flight (register double buffering when 2).
template <int D>
constexpr int decode_prefetch() { return D >= 256 ? 1 : 2; }

template <int D, bool RR = false, bool PF16 = false, bool STUDY = false>
__global__ __launch_bounds__(kDecodeThreads, 1) void miattn_decode_split_kernel(DecodeArgs a) {
  constexpr int NKK = D / 32;   // 16x16x32 steps over the head dim, one 16-B chunk each
  constexpr int NDT = D / 16;   // 16-wide d tiles of the output
  constexpr int PF = decode_prefetch<D>();
  using Smem = DecodeSmem<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Smem::kBytes];

  // 1-D grid: head group fastest, then sequence, split slowest. Workgroups are
  // dealt to the XCDs round robin, so every XCD gets a balanced mix of
  // sequences and split indices, and the (mostly empty) high split indices
  // come last.
  const int HW = a.heads_per_wg;
  const int WPH = kDecodeWaves / HW;                 // waves per kv head
  const int n_hg = a.num_kv_heads / HW;
  const int lin = blockIdx.x;
  // Length-proportional groups (fast path only): the grid is head group
  // fastest, then group index; groups past the plan's last exit.
  const bool balanced = !STUDY && a.balance_units > 0;
  int split, hg, b;
  SplitPlan plan = {0, 0, 0, 0, 0, 1};
  if (balanced) {
    hg = lin % n_hg;
    split = lin / n_hg;
    plan = balanced_plan(a.seq_lens, a.batch, a.max_pages, a.balance_units, split, true);
    // the first workgroup publishes the per-sequence table for the combine
    if (lin == 0 && threadIdx.x < 64)
      write_plan_table(a.seq_lens, a.batch, a.max_pages, plan.group_pages, a.plan_table);
    if (plan.b < 0) return;   // uniform over the workgroup
    b = plan.b;
  } else {
    const int per_split = n_hg * a.batch;
    split = lin / per_split;
    hg = (lin % per_split) % n_hg;
    b = (lin % per_split) / n_hg;
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = hg * HW + wave / WPH;                // this wave's kv head
  const int phase = wave % WPH;                      // this wave's pages: phase + WPH i
  const int tok = lane & 15;     // token row of the S^T A operand
  const int quad = lane >> 4;    // 0..3
  const int hl = lane & 15;      // query head (within the group) owned by this lane
  const int G = a.group;
  const int Hkv = a.num_kv_heads;

  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_pages * kPage ? a.max_pages * kPage : L);
  const int n_pages = (L + kPage - 1) / kPage;
  const int S = a.num_splits;
  // The split's pages in visiting order: its k-th page is logical page
  // logical_page(k) of the sequence, for k < np_split.
  int np_split;
  int p0 = 0;
  if constexpr (!RR) {
    if (balanced) {
      // group plan.s: C consecutive pages (the last group of a sequence fewer)
      const int pps = plan.group_pages;
      p0 = plan.s * pps < n_pages ? plan.s * pps : n_pages;
      np_split = (p0 + pps < n_pages ? p0 + pps : n_pages) - p0;
    } else {
      // every split of every sequence covers the same page budget, sized
      // from the block-table width
      const int pps = (a.max_pages + S - 1) / S;
      p0 = split * pps < n_pages ? split * pps : n_pages;
      const int p1 = p0 + pps < n_pages ? p0 + pps : n_pages;
      np_split = p1 - p0;
    }
  } else {
    const int sh = a.tile_shift;
    const int n_tiles = (n_pages + (1 << sh) - 1) >> sh;
    np_split = 0;
    if (split < n_tiles) {
      const int full = (n_tiles - 1 - split) / S + 1;     // tiles j = split + S r, j < n_tiles
      const int last = split + S * (full - 1);
      const int tail = n_pages - (last << sh);
      np_split = ((full - 1) << sh) + (tail < (1 << sh) ? tail : (1 << sh));
    }
  }
  auto logical_page = [&](int k) -> int {
    if constexpr (!RR) {
      return p0 + k;
    } else {
      const int sh = a.tile_shift;
      return ((split + S * (k >> sh)) << sh) + (k & ((1 << sh) - 1));
    }
  };
  // this wave's i-th page is the split's page phase + WPH i
  const int np = (np_split - phase + WPH - 1) / WPH > 0 ? (np_split - phase + WPH - 1) / WPH : 0;

  // Q^T operand: head hl, d = 32*kk + 8*quad .. +7 (zero for padding heads).
  u32x4 qop[NKK];
  {
    const bool live = hl < G;
    const uint16_t* qp = a.q + ((size_t)b * a.num_q_heads + (size_t)g * G + (live ? hl : 0)) * D + 8 * quad;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qop[kk] = live ? ld16(qp + 32 * kk) : z;
    }
  }

  const size_t row_stride = (size_t)Hkv * D;               // elements between tokens
  const size_t page_stride = (size_t)kPage * row_stride;   // elements between pages
  const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages;

  // Block-table entries of the wave's pages, 64 at a time: lane j holds page
  // j of the current window (-1 if out of range or invalid).
  int bt_win = -1;
  auto load_bt_window = [&](int first) {
    const int i = first + lane;
    int pp = -1;
    if (i < np) {
      pp = bt_row[logical_page(phase + WPH * i)];
      pp = (pp >= 0 && pp < a.num_pages) ? pp : -1;
    }
    bt_win = pp;
  };
  auto phys_page = [&](int i) -> int { return __builtin_amdgcn_readlane(bt_win, i & 63); };

  float m = kNegInf;   // running max (log2 units) for head hl
  float l = 0.f;       // partial running sum over this lane's tokens
  f32x4 acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};

  MIATTN_LDS uint16_t* vstage = (MIATTN_LDS uint16_t*)(smem) + wave * 2 * kPage * Smem::kRowElems;
  MIATTN_LDS uint16_t* kstage = vstage + kPage * Smem::kRowElems;

  // Page copies move whole rows: copy j reads rows RPI j + lrow of the page,
  // CPR 16-byte chunks per row (chunk lch of the row per lane), so each
  // instruction fetches full 128-byte lines. The data is read exactly once,
  // hence non-temporal loads.
  constexpr int CPR = D / 8;         // chunks per row
  constexpr int RPI = 64 / CPR;      // rows per copy; NKK copies cover the 16 rows
  const int lrow = lane / CPR;
  const int lch = lane % CPR;

  // K/V rows of the wave's i-th page into registers; returns the physical
  // page (-1: contributes nothing). The page must lie in the current
  // block-table window. The loads are buffer loads with the page as the
  // buffer (its base uniform, lane offsets inside it), so they never branch:
  // for an invalid page, or a prefetch past the wave's last page (`real`
  // false, uniform), the buffer is empty and every load returns zeros without
  // touching memory; those values are masked (K) or zeroed (V) before use,
  // or never used.
  const uint32_t page_bytes = (uint32_t)(page_stride * 2);
  const uint32_t lane_off = (uint32_t)(((size_t)lrow * row_stride + (size_t)g * D + 8 * lch) * 2);
  auto load_page = [&](int i, bool real, u32x4* kb, u32x4* vb) -> int {
    const int pp = phys_page(i);
    const size_t base = (size_t)(pp >= 0 ? pp : 0) * page_stride;
    const int nrec = (real && pp >= 0) ? (int)page_bytes : 0;
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.k_cache + base), (short)0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.v_cache + base), (short)0, nrec, 0x00020000);
#pragma unroll
    for (int j = 0; j < NKK; ++j) {
      const int o = (int)(lane_off + (uint32_t)(RPI * j * row_stride * 2));
      // cache policy 2: non-temporal, the data is read once
      kb[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, o, 0, 2));
      vb[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, o, 0, 2));
    }
    return pp;
  };

  // Page i's registers into the wave's LDS rows (V rows of tokens past the
  // sequence end or of an invalid page as zeros); the caller may then refill
  // kb/vb.
  auto stage = [&](int i, bool page_ok, const u32x4* kb, const u32x4* vb) {
    const int lp = logical_page(phase + WPH * i);
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < NKK; ++j) {
      const int row = RPI * j + lrow;
      const bool row_ok = page_ok && lp * kPage + row < L;
      lds_st16(kstage + row * Smem::kRowElems + 8 * lch, kb[j]);
      lds_st16(vstage + row * Smem::kRowElems + 8 * lch,
               row_ok ? (PF16 ? bf16x8_to_f16x8(vb[j]) : vb[j]) : z);
    }
  };
  // S^T = K Q^T for the staged page: token tok, d = 32 kk + 8 quad .. +7.
  auto scores = [&]() -> f32x4 {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    const MIATTN_LDS uint16_t* kr = kstage + tok * Smem::kRowElems + 8 * quad;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(lds_ld16(kr + 32 * kk)), as_bf16x8(qop[kk]), s, 0, 0,
                                                  0);
    return s;
  };
  // Online softmax for page i and O^T += V^T P^T from the staged V.
  auto accumulate = [&](int i, f32x4 s, bool page_ok) {
    const int lp = logical_page(phase + WPH * i);
    float t[4];
    float pm = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tk = lp * kPage + 4 * quad + r;
      t[r] = (page_ok && tk < L) ? s[r] * a.c : kNegInf;
      pm = fmaxf(pm, t[r]);
    }
    pm = fmaxf(pm, xor16(pm));
    pm = fmaxf(pm, xor32(pm));
    if (__builtin_amdgcn_ballot_w64(pm > m + kRescaleThreshold)) {
      const float mn = fmaxf(m, pm);
      const float alpha = (m == kNegInf) ? 0.f : exp2_hw(m - mn);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
      m = mn;
    }
    const float mu = (m == kNegInf) ? 0.f : m;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = exp2_hw(t[r] - mu);
    const u32x2 pw = PF16 ? (u32x2){pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3])}
                          : (u32x2){pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
    if (STUDY && a.rounded_l) {
      // the normaliser sums the same rounded weights that enter P.V
      if constexpr (PF16)
        l += (f16lo_to_f32(pw[0]) + f16hi_to_f32(pw[0])) + (f16lo_to_f32(pw[1]) + f16hi_to_f32(pw[1]));
      else
        l += (bf16lo_to_f32(pw[0]) + bf16hi_to_f32(pw[0])) + (bf16lo_to_f32(pw[1]) + bf16hi_to_f32(pw[1]));
    } else {
      l += (p[0] + p[1]) + (p[2] + p[3]);
    }
    const MIATTN_LDS uint16_t* vt = vstage + (4 * quad + (tok >> 2)) * Smem::kRowElems + 4 * (tok & 3);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const u32x2 vw = lds_ld_tr16(vt + 16 * dt);
      if constexpr (PF16)
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, vw), __builtin_bit_cast(f16x4, pw),
                                                        acc[dt], 0, 0, 0);
      else
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_bf16x4(vw), as_bf16x4(pw), acc[dt], 0, 0, 0);
    }
  };

  // Pages are walked in windows of 64 (one block-table entry per lane).
  // Inside a window every load is issued unconditionally: the prefetch past
  // the last page is an empty-buffer load (no memory traffic) and a uniform
  // branch skips its accumulation, so the compiler can count outstanding
  // loads exactly and wait only for the page about to be used.
  for (int w0 = 0; w0 < np; w0 += 64) {
    const int n_in = np - w0 < 64 ? np - w0 : 64;
    load_bt_window(w0);
    u32x4 kb[PF][NKK], vb[PF][NKK];
    int pp_buf[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) pp_buf[j] = load_page(w0 + (j < n_in ? j : n_in - 1), j < n_in, kb[j], vb[j]);
    for (int i0 = 0; i0 < n_in; i0 += PF) {
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        const int ii = i0 + j;                  // index inside the window
        const bool live = ii < n_in;            // uniform
        const bool ok_i = live && pp_buf[j] >= 0;
        stage(w0 + ii, ok_i, kb[j], vb[j]);
        const bool more = ii + PF < n_in;       // uniform: a page is left to fetch
        pp_buf[j] = load_page(w0 + (more ? ii + PF : n_in - 1), more, kb[j], vb[j]);
        if (live) accumulate(w0 + ii, scores(), ok_i);
      }
    }
  }

  // full per-head sum over the four token quads of the wave
  l += xor16(l);
  l += xor32(l);

  if (!STUDY && WPH == 1) {
    // One wave per kv head: the wave holds its heads' whole result, so it
    // normalises and stores it from registers, with no barrier and no LDS
    // round trip (the merge below would weigh it by exp2(0) = 1: the same
    // bits). Lane: query head hl of kv head g, columns 16 dt + 4 quad .. + 3.
    if (hl < G) {
      const bool empty = !(l > 0.f);
      const float inv = empty ? 0.f : 1.f / l;
      const float lse = empty ? kNegInf : (m + log2_hw(l)) * kLn2;
      const size_t row = (size_t)b * a.num_q_heads + (size_t)g * G + hl;
      if (!balanced && S == 1) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const f32x4 o = acc[dt] * inv;
          u32x2 w2 = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          *reinterpret_cast<u32x2*>(a.o + row * D + 16 * dt + 4 * quad) = w2;
        }
        if (a.lse != nullptr && quad == 0) a.lse[row] = lse;
      } else {
        const size_t slot = balanced ? (size_t)(split * a.num_q_heads) + (row - (size_t)b * a.num_q_heads)
                                     : row * S + split;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          *reinterpret_cast<f32x4*>(a.part_o + slot * D + 16 * dt + 4 * quad) = acc[dt] * inv;
        if (quad == 0) a.part_lse[slot] = lse;
      }
    }
    return;
  }

  __syncthreads();   // staging area is reused for the merge below
  float* mo = (float*)smem;                                                // [wave][G][D]
  float* mm = (float*)(smem + (Smem::kBytes - 2 * kDecodeWaves * 16 * 4)); // [wave][16]
  float* ml = mm + kDecodeWaves * 16;                                      // [wave][16]
  if (quad == 0) {
    mm[wave * 16 + hl] = m;
    ml[wave * 16 + hl] = l;
  }
  if (hl < G) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      *reinterpret_cast<f32x4*>(mo + ((size_t)wave * G + hl) * D + 16 * dt + 4 * quad) = acc[dt];
  }
  __syncthreads();

  // merge the WPH waves of each kv head in wave order; one output row per
  // (kv head, query head in its group)
  for (int idx = threadIdx.x; idx < HW * G * (D / 4); idx += kDecodeThreads) {
    const int gh = idx / (G * (D / 4));           // kv head within the workgroup
    const int h = (idx / (D / 4)) % G;
    const int d4 = (idx % (D / 4)) * 4;
    const int w0 = gh * WPH;
    float M = kNegInf;
    for (int w = w0; w < w0 + WPH; ++w) M = fmaxf(M, mm[w * 16 + h]);
    float Lsum = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int w = w0; w < w0 + WPH; ++w) {
      const float mw = mm[w * 16 + h];
      const float f = (mw == kNegInf) ? 0.f : exp2_hw(mw - M);
      Lsum += f * ml[w * 16 + h];
      o += f * *reinterpret_cast<const f32x4*>(mo + ((size_t)w * G + h) * D + d4);
    }
    const bool empty = !(Lsum > 0.f);
    const float inv = empty ? 0.f : 1.f / Lsum;
    const size_t row = (size_t)b * a.num_q_heads + (size_t)(hg * HW + gh) * G + h;
    if (STUDY && a.record != 0) {
      // split statistics: numerator (or normalised partial), reference max,
      // normaliser; an empty split stores (0, -inf, 0)
      f32x4 rec = a.record == 2 ? o * inv : o;
      if (a.record >= 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) rec[e] = round_bf16(rec[e]);
      }
      *reinterpret_cast<f32x4*>(a.part_o + (row * S + split) * D + d4) = rec;
      if (d4 == 0) {
        a.part_m[row * S + split] = empty ? kNegInf : M;
        a.part_l[row * S + split] = empty ? 0.f : Lsum;
      }
      continue;
    }
    o *= inv;
    const float lse = empty ? kNegInf : (M + log2_hw(Lsum)) * kLn2;
    if (!STUDY && !balanced && S == 1) {
      u32x2 w2 = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      *reinterpret_cast<u32x2*>(a.o + row * D + d4) = w2;
      if (a.lse != nullptr && d4 == 0) a.lse[row] = lse;
    } else {
      // partial slot: [row][split], or [group][head] for balanced groups
      const size_t slot = balanced ? (size_t)split * a.num_q_heads + (row - (size_t)b * a.num_q_heads)
                                   : row * S + split;
      *reinterpret_cast<f32x4*>(a.part_o + slot * D + d4) = o;
      if (d4 == 0) a.part_lse[slot] = lse;
    }
  }
}

}  // namespace miattn
