// Tiled prefill forward with an online softmax on gfx950 (bf16 MFMA).
//
// The loop is the FlashAttention forward of "Streaming process" (steps 3-8
// and its code snippet): Q is loaded once, K/V tiles stream through on-chip
// memory while the previous tile is consumed, S = Q K^T lands in fp32
// registers, the row max / exponentials / rescaling run on the vector ALUs,
// P V accumulates into registers, and O / l is cast to bf16 at the end.
//
// MI355X mapping:
//  * Workgroup = 4 waves, one per SIMD. Waves split the NH query heads of one
//    kv-head group (NH: the largest of 4, 2, 1 dividing G) and 4/NH row ranges; each wave owns QB
//    blocks of 32 query rows (the library launches QB = 1), so every K and V
//    operand read from LDS feeds QB MFMAs, and all waves reuse the same K/V
//    tile (GQA sharing of "GPU Datapath", section C).
//  * K/V tiles of Bc = 32*KB keys are double-buffered in LDS and copied
//    straight from HBM into LDS (buffer loads in their LDS form, 16 bytes per
//    lane, whole rows per 16 lanes) one tile ahead, into a swizzled layout
//    that keeps the MFMA operand reads free of bank conflicts; one barrier
//    per tile. Two workgroups share each CU, so one's softmax overlaps the
//    other's matrix-core work.
//  * S^T = K . Q^T on 32x32x16 bf16 MFMAs: lane l owns query row l%32 and 16
//    of every 32 keys (the other 16 sit in lane l^32), so row max and row sum
//    are in-lane reductions plus one v_permlane32_swap.
//  * exp is v_exp_f32 on (s * scale*log2 e - m): one FMA and one exp2 per
//    score. The running max moves only when a tile's max exceeds it by more
//    than 2^8 (exact in real arithmetic; probabilities stay <= 256), so O and
//    l are rescaled only a few times per row.
//  * O^T += V^T . P^T on the same MFMA shape: the accumulator registers of
//    S^T, rounded to bf16, are already the B operand; V^T comes from LDS
//    through ds_read_b64_tr_b16. Lane l then holds all of query row l%32's
//    output columns it owns, so the rescale is a per-lane scalar multiply.
//  * Grid: one workgroup per (kv-head group, query-tile pair, sequence); a
//    workgroup takes query tiles i and n-1-i of its sequence, so every causal
//    workgroup does the same work. The head index varies fastest: workgroups
//    are dealt to the 8 XCDs round robin, so with 8 kv heads each XCD's L2
//    serves one head's K/V; the sequence index varies slowest, so the
//    workgroups resident together read one sequence's K/V.
#pragma once
#include <type_traits>

#include "common.h"

namespace miattn {

struct FwdArgs {
  const uint16_t* q;          // [T, Hq, D]
  const uint16_t* k;          // [T, Hkv, D]; paged: cache [num_pages, 16, Hkv, D]
  const uint16_t* v;
  uint16_t* o;                // [T, Hq, D]
  float* lse;                 // [Hq, T] or null
  const int32_t* cu_seqlens;  // [num_seqs + 1]
  int num_seqs;
  int total_tokens;
  int num_q_heads;
  int num_kv_heads;
  int group;                  // G
  int heads_per_wg;           // NH
  int n_pairs;                // grid units per sequence: query-tile pairs (paged, head_dim 256: query tiles)
  int n_head_slots;           // Hkv * G / NH
  float c;                    // scale * log2(e)
  // paged K/V (chunked prefill): key count per sequence and page table
  const int32_t* seq_lens_k;  // [num_seqs]
  const int32_t* block_table; // [num_seqs, max_pages]
  int max_pages;
  int num_pages;
  // work queue of the head_dim-256 prefill: 8 per-XCD counters and an exit
  // count, all zero when a launch starts (its last workgroup zeroes them)
  unsigned* queue;
};

constexpr float kFwdRescaleThreshold = 8.0f;

// LDS tile of BC rows x D bf16, stored unpadded as 16-byte slots; chunk c of
// row r sits in slot c ^ swz(r). LDS serves 256 bytes (64 banks) per cycle,
// i.e. 16 slots; a row of D = 128 spans all 64 banks, D = 64 half of them.
// K: a 128-bit operand read serves 16 lanes = 16 consecutive rows x one
// chunk per cycle; swz = r mod 16 (D = 64: (r / 2) mod 8, since two rows
// share the banks) puts them in 16 different slots. V: a transposing read
// serves 32 lanes = 4 consecutive rows x 4 consecutive chunks (a 4-aligned
// group) per cycle; swz = 4 (r mod 4) (D = 64: 4 ((r / 2) mod 2)) moves each
// row's group to its own quarter of the banks. Tiles are filled by direct
// HBM->LDS copies of whole rows (16 lanes x 16 B per row for D = 128), so
// the HBM reads stay row-contiguous.
template <int D, int KB>
struct FwdTile {
  static constexpr int BC = 32 * KB;
  static constexpr int CH = D / 8;                      // 16-byte chunks per row
  static constexpr int TILE_BYTES = BC * D * 2;
  static constexpr int NI = TILE_BYTES / 1024 / 4;      // 1-KB direct loads per wave per tile
  static_assert(TILE_BYTES % 4096 == 0, "tile must split into 1-KB loads over 4 waves");
  __device__ static int kswz(int r) { return CH >= 16 ? (r & 15) : ((r >> 1) & (CH - 1)); }
  __device__ static int vswz(int r) { return CH >= 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// QB = 32-row query blocks per wave (1 or 2); KB = 32-key blocks per tile.
// PAGED: keys/values come from a paged cache through the block table, the
// sequence's Lk keys end with its Lq queries (chunked prefill), and causal
// masking aligns the queries to the end: query i sees keys j <= i + Lk - Lq.
template <int D, int QB, int KB, bool CAUSAL, bool PAGED = false, bool F16V = false>
__global__ __launch_bounds__(256, (QB == 1 && D <= 128) ? 2 : 1) void miattn_prefill_fwd_kernel(FwdArgs a) {
  static_assert(!(PAGED && F16V), "the fp16 form of V is made for contiguous V only");
  using TL = FwdTile<D, KB>;
  constexpr int BC = TL::BC;
  constexpr int CH = TL::CH;
  constexpr int NKK = D / 16;   // MFMA steps over the head dim (16 each)
  constexpr int NDT = D / 32;   // 32-wide output column tiles
  // Four distinct LDS objects (K and V, two buffers each): alias analysis can
  // then tell that a direct load in flight into one buffer does not feed reads
  // of another, so reads of the current tile need not wait for the prefetch.
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[TL::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[TL::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[TL::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[TL::TILE_BYTES];
  auto kbuf = [&](int i) { return (MIATTN_LDS uint8_t*)(i == 0 ? k_lds0 : k_lds1); };
  auto vbuf = [&](int i) { return (MIATTN_LDS uint8_t*)(i == 0 ? v_lds0 : v_lds1); };

  const int NH = a.heads_per_wg;
  const int WQ = 4 / NH;
  const int QR = 32 * QB * WQ;   // query rows per tile

  // --- work item: (head slot, tile pair, sequence); head slot fastest ------
  const int lin = blockIdx.x;
  const int hslot = lin % a.n_head_slots;
  const int rest = lin / a.n_head_slots;
  // sequence-major: a sequence's tiles are consecutive, so the workgroups
  // running together on an XCD share that sequence's K/V in its L2
  const int pair = rest % a.n_pairs;
  const int b = rest / a.n_pairs;
  int s0 = a.cu_seqlens[b];
  int s1 = a.cu_seqlens[b + 1];
  s0 = s0 < 0 ? 0 : (s0 > a.total_tokens ? a.total_tokens : s0);
  s1 = s1 < s0 ? s0 : (s1 > a.total_tokens ? a.total_tokens : s1);
  const int Lq = s1 - s0;   // query rows of the sequence
  int Lk = Lq;              // keys of the sequence
  if constexpr (PAGED) {
    Lk = a.seq_lens_k[b];
    Lk = Lk < 0 ? 0 : (Lk > a.max_pages * 16 ? a.max_pages * 16 : Lk);
  }
  const int off = Lk - Lq;  // causal: query i sees keys j <= i + off
  const int n_tiles = (Lq + QR - 1) / QR;
  // Causal tiles i and n-1-i together cost the same for every pair, so a
  // workgroup takes such a pair. With a cached prefix at least as long as
  // the chunk the tiles' costs differ by at most a factor of two and pairing
  // would only double the job size, so the paged grid has one unit per tile
  // and, for such sequences, a workgroup takes one tile, the heaviest first
  // (units past the pairs exit).
  const bool paired = !PAGED || (CAUSAL && off < Lq);
  if (paired ? (pair > n_tiles - 1 - pair) : (pair >= n_tiles)) return;   // uniform over the workgroup
  const int n_mine = (paired && pair != n_tiles - 1 - pair) ? 2 : 1;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hs = wave % NH;
  const int qs = wave / NH;
  const int gpw = a.group / NH;
  const int g = hslot / gpw;
  const int h = g * a.group + (hslot % gpw) * NH + hs;
  const int half = lane >> 5;
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const float c = a.c;

  const size_t kv_row = (size_t)Hkv * D;
  const uint16_t* kbase = a.k + (PAGED ? 0 : (size_t)s0 * kv_row) + (size_t)g * D;
  const uint16_t* vbase = a.v + (PAGED ? 0 : (size_t)s0 * kv_row) + (size_t)g * D;

  // Direct global -> LDS loads of tile kt into buffer `buf` (K and V). Each
  // wave issues NI 1-KB loads per tensor; lane i of load j fills slot
  // lin % CH of row lin / CH (lin = (wave NI + j) 64 + i) with the chunk the
  // swizzle maps there. The address is a uniform tile base plus a fixed
  // per-lane 32-bit offset; on the tail tile rows past the sequence end
  // repeat its last row (their scores are masked, their probabilities 0).
  uint32_t koff[TL::NI], voff[TL::NI];
#pragma unroll
  for (int j = 0; j < TL::NI; ++j) {
    const int lidx = (wave * TL::NI + j) * 64 + lane;
    const int r = lidx / CH;
    const int slot = lidx % CH;
    const size_t rowpart = PAGED ? 0 : (size_t)r * kv_row;   // paged: the row comes per copy
    koff[j] = (uint32_t)((rowpart + 8 * (slot ^ TL::kswz(r))) * 2);
    voff[j] = (uint32_t)((rowpart + 8 * (slot ^ TL::vswz(r))) * 2);
  }
  const uint64_t tile_bytes = (uint64_t)BC * kv_row * 2;
  // Paged: block-table entries [bt_w0, bt_w0 + 64) of this sequence, one per
  // lane (invalid entries read page 0: such inputs never fault, their results
  // are unspecified). A copy instruction covers 64 / CH consecutive rows, all
  // inside one 16-token page, so its page is uniform.
  int bt_w0 = -(1 << 30), bt_win = 0;
  const int32_t* bt_row = a.block_table + (PAGED ? (size_t)b * a.max_pages : 0);
  auto load_tile = [&](int kt, int buf) {
    if constexpr (!PAGED) {
      const bool full = (kt + 1) * BC <= Lk;
      const char* kb0 = (const char*)kbase + (uint64_t)kt * tile_bytes;
      const char* vb0 = (const char*)vbase + (uint64_t)kt * tile_bytes;
#pragma unroll
      for (int j = 0; j < TL::NI; ++j) {
        uint32_t ko = koff[j], vo = voff[j];
        if (!full) {
          const int r = ((wave * TL::NI + j) * 64 + lane) / TL::CH;
          const int rr = kt * BC + r < Lk ? r : Lk - 1 - kt * BC;
          const uint32_t back = (uint32_t)((size_t)(r - rr) * kv_row * 2);
          ko -= back;
          vo -= back;
        }
        dma16_to_lds(kb0, ko, kbuf(buf) + (wave * TL::NI + j) * 1024);
        dma16_to_lds(vb0, vo, vbuf(buf) + (wave * TL::NI + j) * 1024);
      }
    } else {
      // pages of this tile: [kt BC / 16, (kt + 1) BC / 16), clamped to the last
      const int last_page = (Lk - 1) >> 4;
      const int p_lo = (kt * BC) >> 4 < last_page ? (kt * BC) >> 4 : last_page;
      if (p_lo < bt_w0 || p_lo + BC / 16 > bt_w0 + 64) {
        bt_w0 = p_lo;
        const int i = bt_w0 + lane;
        int e = i < a.max_pages ? bt_row[i] : 0;
        bt_win = (e >= 0 && e < a.num_pages) ? e : 0;
      }
#pragma unroll
      for (int j = 0; j < TL::NI; ++j) {
        const int r = ((wave * TL::NI + j) * 64 + lane) / TL::CH;   // row in the tile
        const int r0 = ((wave * TL::NI + j) * 64) / TL::CH;         // first row of this copy
        const int t0 = kt * BC + r0;
        // rows past the last key repeat it (same page: a copy never spans pages)
        const int tl = t0 < Lk ? t0 : Lk - 1;
        const int page = __builtin_amdgcn_readlane(bt_win, (tl >> 4) - bt_w0);
        int t = kt * BC + r;
        t = t < Lk ? t : Lk - 1;
        if (t0 >= Lk) t = Lk - 1;
        const uint64_t pbase = (uint64_t)page * 16 * kv_row * 2;
        const uint32_t rowoff = (uint32_t)((size_t)(t & 15) * kv_row * 2);
        dma16_to_lds((const char*)kbase + pbase, rowoff + koff[j], kbuf(buf) + (wave * TL::NI + j) * 1024);
        dma16_to_lds((const char*)vbase + pbase, rowoff + voff[j], vbuf(buf) + (wave * TL::NI + j) * 1024);
      }
    }
  };

  const int bb = lane >> 4, kq = lane & 15;

  for (int tsel = 0; tsel < n_mine; ++tsel) {
    // a single tile: unit u is tile n - 1 - u, so the launch ends on light
    // tiles
    const int qt = !paired ? n_tiles - 1 - pair : (tsel == 0 ? pair : n_tiles - 1 - pair);
    const int q0 = qt * QR + 32 * QB * qs;   // first query row of this wave

    u32x4 qop[QB][NKK];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = q0 + 32 * qb + (lane & 31);
      const bool ok = row < Lq;
      const uint16_t* qp = a.q + ((size_t)(s0 + (ok ? row : 0)) * Hq + h) * D + 8 * half;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        qop[qb][kk] = ok ? ld16(qp + 16 * kk) : z;
      }
    }

    const int qt_end = qt * QR + QR;
    auto clampk = [&](int x) { return x < 0 ? 0 : (x > Lk ? Lk : x); };
    const int kend_wg = CAUSAL ? clampk(qt_end + off) : Lk;
    const int n_kt = (kend_wg + BC - 1) / BC;
    const int kend_w = CAUSAL ? clampk(q0 + 32 * QB + off) : Lk;
    const int n_kt_w = q0 < Lq ? (kend_w + BC - 1) / BC : 0;   // tiles this wave computes

    float m[QB], l[QB];
    f32x16 acc[QB][NDT];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m[qb] = kNegInf;
      l[qb] = 0.f;
#pragma unroll
      for (int i = 0; i < NDT; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[qb][i][r] = 0.f;
    }

    if (tsel > 0) __syncthreads();   // previous tile's last reads before the buffers are refilled
    if (n_kt > 0) load_tile(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    auto step = [&](int kt, auto bufc) {
      constexpr int buf = decltype(bufc)::value;
      if (kt + 1 < n_kt) load_tile(kt + 1, buf ^ 1);
      if (kt < n_kt_w) {
        const MIATTN_LDS uint8_t* kl = kbuf(buf);
        const MIATTN_LDS uint8_t* vl = vbuf(buf);
        // S^T = K Q^T: lane reads K row 32 kb + lane%32, chunk 2 kk + half
        f32x16 s[QB][KB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int r = 32 * kb + (lane & 31);
          const MIATTN_LDS uint8_t* kr = kl + r * (2 * D);
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            const bf16x8 kop = as_bf16x8(lds_ld16(kr + 16 * ((2 * kk + half) ^ TL::kswz(r))));
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
              s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, as_bf16x8(qop[qb][kk]), s[qb][kb], 0, 0, 0);
          }
        }
        // mask (diagonal / tail tiles only), raw row max, lazy rescale
        const bool need_mask = (kt + 1) * BC > Lk || (CAUSAL && (kt + 1) * BC - 1 > q0 + off);
        if (need_mask) {
          // key of score r in block kb: kt BC + 4 half + (32 kb + 8 (r / 4) + r % 4),
          // kept iff that offset is below lim (compares with immediates, no
          // per-score registers)
          const int kbase_lane = kt * BC + 4 * half;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            int lim = Lk - kbase_lane;
            if (CAUSAL) {
              const int lc = q0 + 32 * qb + (lane & 31) + off + 1 - kbase_lane;
              lim = lc < lim ? lc : lim;
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int r = 0; r < 16; ++r)
                s[qb][kb][r] = (32 * kb + 8 * (r >> 2) + (r & 3)) < lim ? s[qb][kb][r] : kNegInf;
          }
        }
        // P = exp2(s c - m), rounded to bf16 for P.V; the tile's row sum ls
        // adds the fp32 values in score order, then l += ls
        u32x4 pw[QB][KB][2];
        float ls[QB];
        auto exps = [&]() __attribute__((always_inline)) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const float nmu = (m[qb] == kNegInf) ? 0.f : -m[qb];
            ls[qb] = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int r = 0; r < 16; r += 2) {
                const float p0 = exp2_hw(__builtin_fmaf(s[qb][kb][r], c, nmu));
                const float p1 = exp2_hw(__builtin_fmaf(s[qb][kb][r + 1], c, nmu));
                ls[qb] += p0 + p1;
                pw[qb][kb][r >> 3][(r >> 1) & 3] = pack_p<F16V>(p0, p1);
              }
          }
        };
        // lazy rescale: the running max moves only when the tile's max
        // exceeds it by more than 2^8. The tile max is needed only when a
        // probability against the current max could reach that: with a finite
        // max in every lane and every lane's sum at most 2^6, no score is
        // within 2 (log2 units) of the threshold and the probabilities
        // already computed stand. Otherwise (first tile, large or non-finite
        // sums) take the max, apply the rule and recompute
        // (32-key tiles hold too few scores per lane for the check to pay:
        // they always take the max)
        bool unset = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) unset = unset || m[qb] == kNegInf;
        bool slow = KB < 2 || __builtin_amdgcn_ballot_w64(unset) != 0;
        if (!slow) {
          exps();
          bool big = false;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) big = big || !(ls[qb] <= 64.f);
          slow = __builtin_amdgcn_ballot_w64(big) != 0;
        }
        if (slow) {
          float tmax[QB];
          bool grow = false;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            float smax = kNegInf;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int r = 0; r < 16; ++r) smax = fmaxf(smax, s[qb][kb][r]);
            smax = fmaxf(smax, xor32(smax));
            tmax[qb] = smax * c;   // scale > 0, so max(s c) = c max(s)
            grow = grow || (tmax[qb] > m[qb] + kFwdRescaleThreshold);
          }
          if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              const float mn = fmaxf(m[qb], tmax[qb]);
              const float alpha = (m[qb] == kNegInf) ? 0.f : exp2_hw(m[qb] - mn);
              l[qb] *= alpha;
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt) acc[qb][dt] *= alpha;
              m[qb] = mn;
            }
          }
          exps();
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          // O^T += V^T P^T; V^T rows via the transposing read: block bb of
          // 16 lanes reads keys 32kb + 16u + 4(bb/2) + {0..3} (+8), columns
          // 32 dt + 16 (bb%2) + {0..15}
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int r0 = 32 * kb + 16 * u + 4 * (bb >> 1) + (kq >> 2);
            const int r1 = r0 + 8;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
              const int col = 32 * dt + 16 * (bb & 1) + 4 * (kq & 3);   // element column
              const int ch = col >> 3, sub = (col & 7) * 2;             // chunk, byte offset in it
              const u32x2 lo = lds_ld_tr16(vl + r0 * (2 * D) + 16 * (ch ^ TL::vswz(r0)) + sub);
              const u32x2 hi = lds_ld_tr16(vl + r1 * (2 * D) + 16 * (ch ^ TL::vswz(r1)) + sub);
#pragma unroll
              for (int qb = 0; qb < QB; ++qb) acc[qb][dt] = mfma_pv<F16V>(lo, hi, pw[qb][kb][u], acc[qb][dt]);
            }
          }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) l[qb] += ls[qb];
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // tile kt+1 has landed in LDS
      __syncthreads();
    };
    for (int kt = 0; kt < n_kt; kt += 2) {
      step(kt, std::integral_constant<int, 0>{});
      if (kt + 1 < n_kt) step(kt + 1, std::integral_constant<int, 1>{});
    }

    // --- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 --------------------
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float lt = l[qb] + xor32(l[qb]);
      const int qrow = q0 + 32 * qb + (lane & 31);
      if (qrow < Lq) {
        const bool empty = !(lt > 0.f);
        const float inv = empty ? 0.f : 1.f / lt;
        uint16_t* op = a.o + ((size_t)(s0 + qrow) * Hq + h) * D + 4 * half;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x16& A = acc[qb][dt];
            u32x2 w = {pack_bf16x2(A[4 * r4] * inv, A[4 * r4 + 1] * inv),
                       pack_bf16x2(A[4 * r4 + 2] * inv, A[4 * r4 + 3] * inv)};
            *reinterpret_cast<u32x2*>(op + 32 * dt + 8 * r4) = w;
          }
        if (a.lse != nullptr && half == 0)
          a.lse[(size_t)h * a.total_tokens + s0 + qrow] = empty ? kNegInf : (m[qb] + log2_hw(lt)) * kLn2;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs, head_dim 64: the same S^T / O^T orientation on 32x32x2 fp32
// MFMAs with P kept in fp32. Operands are read straight from global memory
// (the fp32 case is the small dense single-head workload; its K/V stay in L2).
// One wave per 32 query rows of one head.
// ---------------------------------------------------------------------------
struct FwdF32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  const int32_t* cu_seqlens;
  int num_seqs;
  int total_tokens;
  int num_q_heads;
  int num_kv_heads;
  int group;
  int n_qtiles;               // ceil(max_seqlen / 32)
  float c;
};

// fp32 prefill (head_dim 64): one workgroup of 8 waves per (query tile of
// 32 rows, head, sequence). The key range is shared out over the waves, tile
// kt to wave kt mod 8, each keeping its own running max, sum and output
// (S^T = K Q^T and O^T += V^T P^T on 32x32x2 fp32 MFMAs, operands straight
// from global memory); the 8 partial states are merged through LDS in wave
// order, so a short sequence's latency is one eighth of its key tiles.
template <bool CAUSAL>
__global__ __launch_bounds__(512) void miattn_prefill_fwd_f32_kernel(FwdF32Args a) {
  constexpr int D = 64;
  constexpr int NW = 8;
  __shared__ f32x4 part[NW][8][64];   // [wave][4-value chunk][lane]
  __shared__ float pm[NW][32], pl[NW][32];
  const int lin = blockIdx.x;
  const int h = lin % a.num_q_heads;
  const int rest = lin / a.num_q_heads;
  const int qt = a.n_qtiles - 1 - rest / a.num_seqs;
  const int b = rest % a.num_seqs;
  int s0 = a.cu_seqlens[b];
  int s1 = a.cu_seqlens[b + 1];
  s0 = s0 < 0 ? 0 : (s0 > a.total_tokens ? a.total_tokens : s0);
  s1 = s1 < s0 ? s0 : (s1 > a.total_tokens ? a.total_tokens : s1);
  const int L = s1 - s0;
  const int q0 = qt * 32;
  if (q0 >= L) return;   // uniform over the workgroup
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int qrow = q0 + (lane & 31);
  const int g = h / a.group;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const size_t kv_row = (size_t)Hkv * D;

  // Q operand: at product step st, lane half `half` supplies d = 32 half +
  // st, so a lane's 32 values are one contiguous 128-byte piece of its row
  // (eight 16-byte loads; one float per lane from scattered rows made every
  // load instruction touch 32-64 cache lines, and the address unit, shared
  // by the workgroup's waves, was the bottleneck). Every operand load reads a
  // valid (clamped) address unconditionally and the value is zeroed
  // afterwards: a load under a condition becomes a branch around it, and the
  // compiler then waits for each load right before its product.
  float qv[32];
  {
    const bool ok = qrow < L;
    const float* qp = a.q + ((size_t)(s0 + (ok ? qrow : 0)) * Hq + h) * D + 32 * half;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(qp + 4 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[4 * i + e] = ok ? t[e] : 0.f;
    }
  }
  const int kend = CAUSAL ? (L < q0 + 32 ? L : q0 + 32) : L;
  float m = kNegInf, l = 0.f;
  f32x16 acc[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) { acc[0][r] = 0.f; acc[1][r] = 0.f; }
  const float* kb = a.k + (size_t)s0 * kv_row + (size_t)g * D;
  const float* vb = a.v + (size_t)s0 * kv_row + (size_t)g * D;

  for (int k0 = 32 * wave; k0 < kend; k0 += 32 * NW) {
    // V operands of the tile, loaded first so their latency overlaps S:
    // step r pairs key 8(r/4) + r%4 (lanes < 32) with key + 4
    float vv[16][2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + 8 * (r >> 2) + 4 * half + (r & 3);
      const bool ok = key < L;
      const float* vp = vb + (size_t)(ok ? key : 0) * kv_row + (lane & 31);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) vv[r][dt] = vp[32 * dt];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) vv[r][dt] = ok ? vv[r][dt] : 0.f;
    }
    // S^T (32 keys x 32 queries); A = K (row key k0 + lane%32, col d = 32 half + st)
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    const int krow = k0 + (lane & 31);
    const bool kok = krow < L;
    const float* kp = kb + (size_t)(kok ? krow : 0) * kv_row + 32 * half;
    float kv[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(kp + 4 * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) kv[4 * i + e] = t[e];
    }
    __builtin_amdgcn_sched_barrier(0);   // all of the tile's loads issued before the products
#pragma unroll
    for (int st = 0; st < 32; ++st)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(kok ? kv[st] : 0.f, qv[st], s, 0, 0, 0);
    float tmax = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + 8 * (r >> 2) + 4 * half + (r & 3);
      const bool ok = key < L && (!CAUSAL || key <= qrow);
      s[r] = ok ? s[r] * a.c : kNegInf;
      tmax = fmaxf(tmax, s[r]);
    }
    tmax = fmaxf(tmax, xor32(tmax));
    const float mn = fmaxf(m, tmax);
    const float alpha = (m == kNegInf) ? 0.f : exp2_hw(m - mn);
    l *= alpha;
    acc[0] *= alpha;
    acc[1] *= alpha;
    m = mn;
    const float mu = (m == kNegInf) ? 0.f : m;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = exp2_hw(s[r] - mu);
      l += s[r];
    }
    // O^T += V^T P^T
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv[r][dt], s[r], acc[dt], 0, 0, 0);
  }
  l += xor32(l);

  // merge: wave w combines value chunk w (row lane % 32, d = 32 (w / 4) +
  // 8 (w % 4) + 4 half + 0..3) of the 8 partial states, in wave order
  if (lane < 32) {
    pm[wave][lane] = m;
    pl[wave][lane] = l;
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const f32x16& A = acc[c >> 2];
    part[wave][c][lane] = (f32x4){A[4 * (c & 3)], A[4 * (c & 3) + 1], A[4 * (c & 3) + 2], A[4 * (c & 3) + 3]};
  }
  __syncthreads();
  const int row = lane & 31;
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, pm[w][row]);
  float lt = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float mw = pm[w][row];
    const float f = (mw == kNegInf) ? 0.f : exp2_hw(mw - M);
    lt += f * pl[w][row];
    o += f * part[w][wave][lane];
  }
  if (qrow < L) {
    const bool empty = !(lt > 0.f);
    const float inv = empty ? 0.f : 1.f / lt;
    float* op = a.o + ((size_t)(s0 + qrow) * Hq + h) * D + 32 * (wave >> 2) + 8 * (wave & 3) + 4 * half;
    *reinterpret_cast<f32x4*>(op) = o * inv;
    if (a.lse != nullptr && wave == 0 && half == 0)
      a.lse[(size_t)h * a.total_tokens + s0 + qrow] = empty ? kNegInf : (M + log2_hw(lt)) * kLn2;
  }
}

}  // namespace miattn
