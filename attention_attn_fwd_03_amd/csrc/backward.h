// Attention backward by recomputation on gfx950 (bf16 in and out, fp16 MFMA).
//
// The backward pass sketched in the ELI5 of "Why your local LLM feels dumber
// than it is" does not keep the score matrix: it recomputes the scores tile by
// tile from Q, K and the forward's log-sum-exp, exactly as the forward made
// them. With s = scale q.k, P = exp(s - LSE) and the upstream gradient dO:
//     dV_j = sum_i P_ij dO_i,      dP_ij = dO_i . V_j,
//     dS_ij = P_ij (dP_ij - Delta_i),   Delta_i = dO_i . O_i  (= sum_j P_ij dP_ij),
//     dQ_i = scale sum_j dS_ij K_j,      dK_j = scale sum_i dS_ij Q_i.
// Three kernels, all with fixed reduction orders (bitwise reproducible, no
// atomics):
//  * prep: Delta = rowsum(dO * O) in fp32, the LSE in log2 units (both in
//    rows padded by 32 so tile-sized copies stay in bounds), and fp16 copies
//    of Q, dO, K and V, in one pass over the inputs.
//  * dK/dV: one workgroup of 8 waves per (kv head, 64 keys, sequence), two
//    per SIMD: the two waves of a SIMD take 32 keys each and share a
//    double-buffered Q/dO tile pair copied straight from HBM into LDS, and
//    the four pairs take every fourth (query head, 32-query tile) step of the
//    group; the four partial sums of each key are added through LDS in a
//    fixed order at the end. Per tile: S = Q K^T and dP = dO V^T (query rows,
//    key columns), then dV^T += dO^T P and dK^T += Q^T dS: the accumulator
//    registers of P and dS, rounded to fp16, are the B operand as they
//    stand; dO^T and Q^T come from the same LDS tile through the transposing
//    read. At head_dim 256 four waves share each Q/dO tile and split 64 keys,
//    16 each (miattn_bwd_dkdv_d256_kernel).
//  * dQ: the forward's orientation: one wave per 32 query rows of one head,
//    S^T = K Q^T and dP^T = V dO^T with Q, dO held as operands, K/V tiles
//    streaming through LDS, dQ^T += K^T dS^T with K^T read transposed.
// dQ is not accumulated inside the dK/dV kernel, which would need atomics or
// an ordering between workgroups: the dQ kernel recomputes S and dP instead
// (7 products per key/query pair instead of 5).
// Operands are fp16, not bf16: the bf16 inputs convert exactly (inside fp16's
// range), and P and dS then round to fp16 (11 significant bits) instead of
// bf16 (8) for the three gradient products. The gradients are unbounded sums
// of such products; with bf16 P and dS their rounding alone exceeds the bf16
// output bar for magnitudes above ~2.
#pragma once
#include <type_traits>

#include "common.h"

namespace miattn {

struct BwdArgs {
  const uint16_t* q;          // [T, Hq, D] bf16
  const uint16_t* k;          // [T, Hkv, D] bf16
  const uint16_t* v;
  const uint16_t* o;          // [T, Hq, D] forward output, bf16
  const uint16_t* dout;       // [T, Hq, D] bf16
  const float* lse;           // [Hq, T] forward log-sum-exp (natural log)
  float* stats;               // workspace [2][Hq][t_pad]: LSE in log2 units, Delta
  uint16_t* q16;              // workspace fp16 copies: [T, Hq, D]
  uint16_t* do16;             // [T, Hq, D]
  uint16_t* k16;              // [T, Hkv, D]
  uint16_t* v16;              // [T, Hkv, D]
  uint16_t* dq;               // [T, Hq, D] bf16
  uint16_t* dk;               // [T, Hkv, D] bf16
  uint16_t* dv;
  const int32_t* cu_seqlens;  // [num_seqs + 1]
  int num_seqs;
  int total_tokens;
  int t_pad;                  // row length of the stats arrays (>= T + 32)
  int num_q_heads;
  int num_kv_heads;
  int group;                  // G
  int heads_per_wg;           // dQ kernel: query heads per workgroup (NH)
  int n_head_slots;           // dQ kernel: Hkv * G / NH
  int n_kblocks;              // dK/dV grid: key blocks per sequence (32 keys; 64 at head_dim 256)
  int n_qunits;               // dQ grid: query tiles per sequence
  float c;                    // scale * log2(e)
  float scale;
};

// LDS tile of R rows x D 16-bit values read both ways: as a 128-bit operand
// (16 consecutive rows x one 16-byte chunk per cycle) and through the
// transposing read (4 consecutive rows x 4 consecutive chunks per cycle).
// Chunk c of row r sits in slot c ^ swz(r). D >= 128 (16+ slots per row, one
// row per 64 banks): swz = 4 (r mod 4) + (r / 4) mod 4 gives 16 consecutive
// rows 16 different slots, and 4 consecutive rows 4 different groups of 4
// slots. D = 64 (two rows per 64 banks): the same on r / 2, with the parity
// of r choosing the half of the banks.
template <int D>
struct BwdTile {
  static constexpr int CH = D / 8;
  __device__ static int swz(int r) {
    return CH >= 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
};

// Forward log-sum-exp in log2 units of the raw score times c; a row that saw
// no key (-inf) gives +inf, i.e. P = 0.
__device__ __forceinline__ float lse_to_log2(float lse) {
  return lse == kNegInf ? __builtin_inff() : lse * kLog2e;
}

// ---------------------------------------------------------------- prep
// Rows (token, query head) give Delta = dO . O in fp32, the LSE in log2 units
// and fp16 copies of Q and dO; rows (token, kv head) give fp16 copies of K and
// V. CH = D/8 lanes per row, 16 bytes each; a row group never straddles the
// two ranges' boundary branch (the branch is uniform over the CH lanes).
template <int D>
__global__ __launch_bounds__(256) void miattn_bwd_prep_kernel(BwdArgs a) {
  constexpr int CH = D / 8;
  constexpr int RPB = 256 / CH;
  const int t = threadIdx.x;
  const long row = (long)blockIdx.x * RPB + t / CH;
  const long rq = (long)a.total_tokens * a.num_q_heads;
  const long rk = (long)a.total_tokens * a.num_kv_heads;
  const int ch = t % CH;
  if (row < rq) {
    const size_t e = (size_t)row * D + 8 * ch;
    const u32x4 ov = ld16(a.o + e);
    const u32x4 dv = ld16(a.dout + e);
    st16(a.q16 + e, bf16x8_to_f16x8(ld16(a.q + e)));
    st16(a.do16 + e, bf16x8_to_f16x8(dv));
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += bf16lo_to_f32(ov[i]) * bf16lo_to_f32(dv[i]);
      acc += bf16hi_to_f32(ov[i]) * bf16hi_to_f32(dv[i]);
    }
#pragma unroll
    for (int m = CH / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, CH);
    if (ch == 0) {
      const long tok = row / a.num_q_heads;
      const int h = (int)(row % a.num_q_heads);
      const size_t si = (size_t)h * a.t_pad + tok;
      a.stats[si] = lse_to_log2(a.lse[(size_t)h * a.total_tokens + tok]);
      a.stats[(size_t)a.num_q_heads * a.t_pad + si] = acc;
    }
  } else if (row < rq + rk) {
    const size_t e = (size_t)(row - rq) * D + 8 * ch;
    st16(a.k16 + e, bf16x8_to_f16x8(ld16(a.k + e)));
    st16(a.v16 + e, bf16x8_to_f16x8(ld16(a.v + e)));
  }
}

// ---------------------------------------------------------------- dK / dV, head_dim 64 and 128
// Two waves per SIMD. (With four waves that each own a double-buffered Q/dO
// tile pair, the LDS, 146 KB, and the registers, 328, allow one.) A
// workgroup of eight waves covers 64 keys; waves p and p + 4 run on the same
// SIMD, take keys 0-31 and 32-63 of the block, and walk the same steps p,
// p + 4, ... of the group's (query head, 32-query tile) list, so they share one
// double-buffered Q/dO tile pair, each copying half of it. Every wave holds
// the dV^T, dK^T accumulators of its 32 keys and their V operands in
// registers and reads the K operands from LDS (the 64 keys' K sit there for
// the whole loop), which brings it to two waves per SIMD. The pairs keep
// step with one workgroup barrier per step; a step whose queries all precede
// a wave's keys (causal) is skipped by that wave. The four partial sums of
// each 32-key half are added in pair order, one half after the other, through
// the Q/dO buffers.
// Per step: S = Q K^T and dP = dO V^T (query rows, key columns), then
// dV^T += dO^T P and dK^T += Q^T dS with P and dS, rounded to fp16, taken
// from the accumulators as B operands as they stand and dO^T, Q^T read from
// the same LDS tile through the transposing read. The tile swizzle serves
// both read shapes (BwdTile).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void miattn_bwd_dkdv_pair_kernel(BwdArgs a) {
  using TL = BwdTile<D>;
  constexpr int CH = TL::CH;
  constexpr int NKK = D / 16;                        // MFMA steps over the head dim
  constexpr int NDT = D / 32;                        // 32-wide d blocks of dK^T / dV^T
  constexpr int QT = 32;                             // queries per tile
  constexpr int TILE = QT * D * 2;                   // bytes of one 32-row tile
  constexpr int NC = TILE / 1024;                    // 1-KB copies per tile
  constexpr int NCH = NC / 2;                        // ... issued by each wave of a pair
  static_assert(NC % 2 == 0, "a tile must split into 1-KB copies over two waves");
  static_assert(2 * QT * D * 4 <= 4 * TILE, "two pairs' fp32 partials must fit one tile array");
  // [pair] tiles; four distinct LDS objects, so that a copy in flight into
  // one buffer does not hold up reads of the other
  __shared__ __attribute__((aligned(1024))) uint8_t q_lds0[4 * TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t q_lds1[4 * TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t d_lds0[4 * TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t d_lds1[4 * TILE];
  __shared__ __attribute__((aligned(16))) float st_lds0[4 * 64];   // per pair: 32 LSE, 32 Delta
  __shared__ __attribute__((aligned(16))) float st_lds1[4 * 64];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds[2 * TILE];   // K of the 64 keys

  // work item: (kv head, 64-key block, sequence), kv head fastest, sequence
  // slowest; key block 0 (the most causal work) first
  const int lin = blockIdx.x;
  const int g = lin % a.num_kv_heads;
  const int rest = lin / a.num_kv_heads;
  const int kblk = rest % a.n_kblocks;
  const int b = rest / a.n_kblocks;
  int s0 = a.cu_seqlens[b];
  int s1 = a.cu_seqlens[b + 1];
  s0 = s0 < 0 ? 0 : (s0 > a.total_tokens ? a.total_tokens : s0);
  s1 = s1 < s0 ? s0 : (s1 > a.total_tokens ? a.total_tokens : s1);
  const int L = s1 - s0;
  const int kb0 = kblk * 64;
  if (kb0 >= L) return;   // uniform over the workgroup

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pr = wave & 3;         // the pair (and SIMD)
  const int kh = wave >> 2;        // the pair's key half
  const int half = lane >> 5;
  const int bb = lane >> 4, kq = lane & 15;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = a.group;
  const float c = a.c;
  const int kw0 = kb0 + 32 * kh;                     // this wave's first key
  const int key = kw0 + (lane & 31);                 // this lane's key column
  const bool key_ok = key < L;

  const uint32_t qaddr0 = (uint32_t)(uintptr_t)((MIATTN_LDS uint8_t*)q_lds0 + pr * TILE);
  const uint32_t qaddr1 = (uint32_t)(uintptr_t)((MIATTN_LDS uint8_t*)q_lds1 + pr * TILE);
  const uint32_t daddr0 = (uint32_t)(uintptr_t)((MIATTN_LDS uint8_t*)d_lds0 + pr * TILE);
  const uint32_t daddr1 = (uint32_t)(uintptr_t)((MIATTN_LDS uint8_t*)d_lds1 + pr * TILE);
  const uint32_t saddr0 = (uint32_t)(uintptr_t)((MIATTN_LDS float*)st_lds0 + pr * 64);
  const uint32_t saddr1 = (uint32_t)(uintptr_t)((MIATTN_LDS float*)st_lds1 + pr * 64);

  // K of the 64 keys into k_lds and their V into q_lds1 (which no step fills
  // before the loop starts), swizzled like the Q/dO tiles; keys past the
  // sequence end repeat its last key (their P and dS are masked to 0)
  {
    const size_t kv_row = (size_t)Hkv * D;
    const char* ksrc = (const char*)(a.k16 + (size_t)(s0 + kb0) * kv_row + (size_t)g * D);
    const char* vsrc = (const char*)(a.v16 + (size_t)(s0 + kb0) * kv_row + (size_t)g * D);
#pragma unroll
    for (int j = wave; j < 2 * NC; j += 8) {
      const int lidx = j * 64 + lane;
      const int r = lidx / CH;
      const int slot = lidx % CH;
      const int rr = kb0 + r < L ? r : L - 1 - kb0;
      const uint32_t off = (uint32_t)(((size_t)rr * kv_row + 8 * (slot ^ TL::swz(r))) * 2);
      dma16_to_lds(ksrc, off, (MIATTN_LDS uint8_t*)k_lds + j * 1024);
      dma16_to_lds(vsrc, off, (MIATTN_LDS uint8_t*)q_lds1 + j * 1024);
    }
  }
  const MIATTN_LDS uint8_t* k_l = (const MIATTN_LDS uint8_t*)k_lds;

  // steps: (query tile, query head of the group), the last query tile first
  // and the heads fastest, down to (causal) the tile holding query kb0; pair p
  // takes steps p, p + 4, ... Every key block walks the same tiles in the
  // same order, so the workgroups resident on an XCD read one query tile at a
  // time and share it in L2 (a head-by-head walk from each block's own first
  // tile spread them over the group's whole Q/dO, 8 MB at 4K tokens).
  const int n_qt = (L + QT - 1) / QT;
  const int qt0 = CAUSAL ? kb0 / QT : 0;
  const int nq = n_qt - qt0;
  const int n_steps = G * nq;
  const int n_mine = n_steps > pr ? (n_steps - pr + 3) / 4 : 0;
  const int n_iter = (n_steps + 3) / 4;             // pair 0's count, the most

  // copy j of a tile (this wave: j = kh NCH .. kh NCH + NCH - 1): lane fills
  // slot lidx % CH of row lidx / CH (lidx = 64 j + lane) with the chunk the
  // swizzle maps there; rows past the sequence end repeat its last row
  const size_t q_row = (size_t)Hq * D;
  uint32_t qoff[NCH];
#pragma unroll
  for (int jj = 0; jj < NCH; ++jj) {
    const int lidx = (kh * NCH + jj) * 64 + lane;
    const int r = lidx / CH;
    const int slot = lidx % CH;
    qoff[jj] = (uint32_t)(((size_t)r * q_row + 8 * (slot ^ TL::swz(r))) * 2);
  }
  // LSE (lanes 0-7) and Delta (lanes 8-15) of the tile's 32 rows, copied by
  // the pair's first wave
  const uint32_t st_lane = (uint32_t)(((lane >= 8 ? (size_t)Hq * a.t_pad : 0) + 4 * (lane & 7)) * 4);
  auto load_tile = [&](int i, int buf) {
    const int st = pr + 4 * i;
    const int h = g * G + st % G;
    const int q0 = (n_qt - 1 - st / G) * QT;
    const bool full = q0 + QT <= L;
    const char* qsrc = (const char*)(a.q16 + ((size_t)(s0 + q0) * Hq + h) * D);
    const char* dsrc = (const char*)(a.do16 + ((size_t)(s0 + q0) * Hq + h) * D);
#pragma unroll
    for (int jj = 0; jj < NCH; ++jj) {
      const int j = kh * NCH + jj;
      uint32_t off = qoff[jj];
      if (!full) {
        const int r = (j * 64 + lane) / CH;
        const int rr = q0 + r < L ? r : L - 1 - q0;
        off -= (uint32_t)((size_t)(r - rr) * q_row * 2);
      }
      dma16_to_lds_asm(qsrc, off, (buf ? qaddr1 : qaddr0) + j * 1024);
      dma16_to_lds_asm(dsrc, off, (buf ? daddr1 : daddr0) + j * 1024);
    }
    if (kh == 0 && lane < 16)
      dma16_to_lds_asm(a.stats, st_lane + (uint32_t)(((size_t)h * a.t_pad + s0 + q0) * 4), buf ? saddr1 : saddr0);
  };

  f32x16 dk_acc[NDT], dv_acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk_acc[i][r] = 0.f;
      dv_acc[i][r] = 0.f;
    }

  if (n_mine > 0) load_tile(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();   // K, V of the block and every pair's first tile are in LDS

  // this wave's 32 keys' V operands stay in registers (lane: key lane%32,
  // d = 16 kk + 8 half + 0..7); the barrier after the reads frees q_lds1
  u32x4 vreg[NKK];
  const int kr_l = 32 * kh + (lane & 31);            // this lane's key row in the block
  {
    const MIATTN_LDS uint8_t* v_l = (const MIATTN_LDS uint8_t*)q_lds1;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) vreg[kk] = lds_ld16(v_l + kr_l * (2 * D) + 16 * ((2 * kk + half) ^ TL::swz(kr_l)));
  }
  __syncthreads();

  // LDS operand addresses: a per-lane part plus a per-lane XOR term against a
  // compile-time offset. The swizzle of a row depends on its low bits only,
  // so K rows 32 kh + r share Q's terms. Operand reads: chunk 2 kk + half of
  // row r is 32 (kk ^ (sw >> 1)) + 16 (half ^ (sw & 1)). Transposing reads:
  // rows r0 = 16 u + 4 (bb / 2) + kq / 4 and r0 + 8, chunk 4 dt + c0; with
  // sw(r0) = 4 ta + tb (ta the same for both rows) the chunk's slot is
  // 4 (dt ^ ta) + (c0 ^ tb).
  uint32_t n_lane, n_x, k_lane, t_lane0, t_lane1, t_x;
  {
    const int r = lane & 31;
    const int sw = TL::swz(r);
    n_lane = (uint32_t)(r * (2 * D) + 16 * (half ^ (sw & 1)));
    k_lane = (uint32_t)(kr_l * (2 * D) + 16 * (half ^ (sw & 1)));
    n_x = (uint32_t)(32 * (sw >> 1));
    const int r0 = 4 * (bb >> 1) + (kq >> 2), r1 = r0 + 8;
    const int c0 = 2 * (bb & 1) + ((kq & 3) >> 1);
    const int sub = 8 * (kq & 1);
    const int s0w = TL::swz(r0), s1w = TL::swz(r1);
    t_lane0 = (uint32_t)(r0 * (2 * D) + 16 * (c0 ^ (s0w & 3)) + sub);
    t_lane1 = (uint32_t)(r1 * (2 * D) + 16 * (c0 ^ (s1w & 3)) + sub);
    t_x = (uint32_t)(64 * (s0w >> 2));
  }
  // one loop body for both buffers (a copy per buffer would give the
  // accumulators a different register home in each and copies between them)
  for (int i = 0; i < n_iter; ++i) {
    const int buf = i & 1;
    const int st = pr + 4 * i;
    const int q0 = (n_qt - 1 - st / G) * QT;
    // a causal step whose queries all precede this wave's keys adds nothing
    const bool work = i < n_mine && !(CAUSAL && q0 + QT <= kw0);
    const MIATTN_LDS uint8_t* ql = (const MIATTN_LDS uint8_t*)(uintptr_t)(buf ? qaddr1 : qaddr0);
    const MIATTN_LDS uint8_t* dl_ = (const MIATTN_LDS uint8_t*)(uintptr_t)(buf ? daddr1 : daddr0);
    const MIATTN_LDS float* sl = (const MIATTN_LDS float*)(uintptr_t)(buf ? saddr1 : saddr0);
    // S = Q K^T and dP = dO V^T: A = row lane%32 of the tile, chunk 2 kk + half
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.f;
      dp[r] = 0.f;
    }
    if (work) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const uint32_t x = ((uint32_t)(32 * kk)) ^ n_x;
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(lds_ld16(ql + n_lane + x)), as_f16x8(lds_ld16(k_l + k_lane + x)), s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(lds_ld16(dl_ + n_lane + x)), as_f16x8(vreg[kk]), dp, 0, 0, 0);
      }
    }
    // The next step's copies go out after the products above: at head_dim
    // 128 the kernel runs at the 256-register limit with a few values
    // spilled, and a reload of one waits for every memory load issued before
    // it, copies included.
    if (i + 1 < n_mine) load_tile(i + 1, buf ^ 1);
    if (work) {
      // P = exp2(s c - lse2) and dS = P (dP - Delta), 0 outside the sequence
      // and (causal) above the diagonal: a masked score becomes -inf, so P = 0
      // (a row's LSE in log2 units is finite, or +inf for a row that saw no
      // key) and dS = 0 (dP and Delta finite); rows past the sequence end,
      // whose stats rows may hold anything, take LSE = Delta = 0
      const bool need_mask = kw0 + 32 > L || q0 + QT > L || (CAUSAL && kw0 + 31 > q0);
      if (need_mask) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int qrow = q0 + 8 * (e >> 2) + 4 * half + (e & 3);
          const bool okm = key_ok & (qrow < L) & (!CAUSAL | (key <= qrow));
          s[e] = okm ? s[e] : kNegInf;
        }
      }
      const bool tail = q0 + QT > L;
      u32x4 pw[2], dsw[2];
      // this lane's 16 rows: 8 (e/4) + 4 half + e%4, four at a time
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        f32x4 lv = *reinterpret_cast<const MIATTN_LDS f32x4*>(sl + 8 * gi + 4 * half);
        f32x4 dv = *reinterpret_cast<const MIATTN_LDS f32x4*>(sl + 32 + 8 * gi + 4 * half);
        if (tail) {
          const int rem = L - (q0 + 8 * gi + 4 * half);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lv[e] = e < rem ? lv[e] : 0.f;
            dv[e] = e < rem ? dv[e] : 0.f;
          }
        }
#pragma unroll
        for (int e1 = 0; e1 < 4; e1 += 2) {
          const int e0 = 4 * gi + e1;
          const float p0 = exp2_hw(__builtin_fmaf(s[e0], c, -lv[e1]));
          const float p1 = exp2_hw(__builtin_fmaf(s[e0 + 1], c, -lv[e1 + 1]));
          pw[e0 >> 3][(e0 >> 1) & 3] = pack_f16x2(p0, p1);
          dsw[e0 >> 3][(e0 >> 1) & 3] = pack_f16x2(p0 * (dp[e0] - dv[e1]), p1 * (dp[e0 + 1] - dv[e1 + 1]));
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS; X^T rows through the transposing
      // read: block bb of 16 lanes reads rows 16 u + 4 (bb / 2) + {0..3} (+8),
      // columns 32 dt + 16 (bb % 2) + {0..15}
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const uint32_t x = ((uint32_t)(64 * dt)) ^ t_x;
          const uint32_t u0 = 16 * u * (2 * D);
          const f16x8 dot = as_f16x8(lds_ld_tr16(dl_ + t_lane0 + u0 + x), lds_ld_tr16(dl_ + t_lane1 + u0 + x));
          const f16x8 qtr = as_f16x8(lds_ld_tr16(ql + t_lane0 + u0 + x), lds_ld_tr16(ql + t_lane1 + u0 + x));
          dv_acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(dot, as_f16x8(pw[u]), dv_acc[dt], 0, 0, 0);
          dk_acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(qtr, as_f16x8(dsw[u]), dk_acc[dt], 0, 0, 0);
        }
      }
    }
    // this wave's copies for step i + 1 have landed; the barrier publishes
    // both halves and closes the reads of buffer buf
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // the four partials of key half 0, then of half 1, added in pair order:
  // pair p's dK^T / dV^T go to [key][d] fp32 in the tile arrays (dK: q_lds,
  // dV: d_lds; pairs 0-1 in buffer 0, 2-3 in buffer 1)
  const float sc = a.scale;
#pragma unroll 1
  for (int rnd = 0; rnd < 2; ++rnd) {
    if (rnd > 0) __syncthreads();   // half 0's sums have been read
    if (kh == rnd) {
      MIATTN_LDS float* kp = (MIATTN_LDS float*)(pr < 2 ? q_lds0 : q_lds1) + (pr & 1) * QT * D;
      MIATTN_LDS float* vp = (MIATTN_LDS float*)(pr < 2 ? d_lds0 : d_lds1) + (pr & 1) * QT * D;
      const int kr = lane & 31;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = 32 * dt + 8 * r4 + 4 * half;
          f32x4 wk = {dk_acc[dt][4 * r4], dk_acc[dt][4 * r4 + 1], dk_acc[dt][4 * r4 + 2], dk_acc[dt][4 * r4 + 3]};
          f32x4 wv = {dv_acc[dt][4 * r4], dv_acc[dt][4 * r4 + 1], dv_acc[dt][4 * r4 + 2], dv_acc[dt][4 * r4 + 3]};
          *reinterpret_cast<MIATTN_LDS f32x4*>(kp + kr * D + d0) = wk;
          *reinterpret_cast<MIATTN_LDS f32x4*>(vp + kr * D + d0) = wv;
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < QT * (D / 4); idx += 512) {
      const int kr = idx / (D / 4);
      const int d0 = 4 * (idx % (D / 4));
      const int kk_ = kb0 + 32 * rnd + kr;
      if (kk_ >= L) continue;
      const int eo = kr * D + d0;
      const f32x4 k0 = *reinterpret_cast<const MIATTN_LDS f32x4*>((MIATTN_LDS float*)q_lds0 + eo);
      const f32x4 k1 = *reinterpret_cast<const MIATTN_LDS f32x4*>((MIATTN_LDS float*)q_lds0 + QT * D + eo);
      const f32x4 k2 = *reinterpret_cast<const MIATTN_LDS f32x4*>((MIATTN_LDS float*)q_lds1 + eo);
      const f32x4 k3 = *reinterpret_cast<const MIATTN_LDS f32x4*>((MIATTN_LDS float*)q_lds1 + QT * D + eo);
      const f32x4 v0 = *reinterpret_cast<const MIATTN_LDS f32x4*>((MIATTN_LDS float*)d_lds0 + eo);
      const f32x4 v1 = *reinterpret_cast<const MIATTN_LDS f32x4*>((MIATTN_LDS float*)d_lds0 + QT * D + eo);
      const f32x4 v2 = *reinterpret_cast<const MIATTN_LDS f32x4*>((MIATTN_LDS float*)d_lds1 + eo);
      const f32x4 v3 = *reinterpret_cast<const MIATTN_LDS f32x4*>((MIATTN_LDS float*)d_lds1 + QT * D + eo);
      const f32x4 ks = (((k0 + k1) + k2) + k3) * sc;
      const f32x4 vs = ((v0 + v1) + v2) + v3;
      const size_t go = ((size_t)(s0 + kk_) * Hkv + g) * D + d0;
      u32x2 wk = {pack_bf16x2(ks[0], ks[1]), pack_bf16x2(ks[2], ks[3])};
      u32x2 wv = {pack_bf16x2(vs[0], vs[1]), pack_bf16x2(vs[2], vs[3])};
      *reinterpret_cast<u32x2*>(a.dk + go) = wk;
      *reinterpret_cast<u32x2*>(a.dv + go) = wv;
    }
  }
}

// ---------------------------------------------------------------- dK / dV, head_dim 256
// At head_dim 256 the form above does not fit: each wave's double-buffered
// 32-row Q and dO tiles are 16 KB apiece (256 KB of LDS for four waves), and
// dK^T, dV^T of 32 keys take 256 accumulator registers. Here the four waves of
// a workgroup share one double-buffered Q/dO tile and split the workgroup's 64
// keys, 16 each, on 16x16x32 MFMAs: dK^T and dV^T of 16 keys are 16 blocks of
// 16 x 16 each (128 registers), the 16 keys' K and V operands stay in
// registers, and every (query head, 32-query tile) step of the group is taken
// by all four waves between two workgroup barriers. Each key belongs to one
// wave, so the sums need no merge across waves.
// Lane l (c = l mod 16, j = l / 16) in the 16x16x32 products: A holds row c and
// k-elements 8j..8j+7, B column c and the same k-elements, the result column c
// and rows 4j..4j+3. With k over the 32 queries of a tile, element m of a
// lane's eight stands for query 16 (m / 4) + 4j + m mod 4, which is where the
// two 16-query blocks of S leave a lane's P values; the dO^T and Q^T operands
// read the same queries through the transposing LDS read.
template <bool CAUSAL>
__global__ __launch_bounds__(256, 1) void miattn_bwd_dkdv_d256_kernel(BwdArgs a) {
  constexpr int D = 256;
  using TL = BwdTile<D>;
  constexpr int CH = TL::CH;                         // 16-byte chunks per row
  constexpr int QT = 32;                             // queries per tile
  constexpr int KW = 16;                             // keys per wave
  constexpr int TILE = QT * D * 2;                   // bytes of one Q or dO tile
  constexpr int NC = TILE / 1024;                    // 1-KB copies per tensor and tile
  constexpr int NCW = NC / 4;                        // ... issued by each wave
  constexpr int NKS = D / 32;                        // 16x16x32 steps over the head dim
  constexpr int NDB = D / 16;                        // 16-row blocks of dK^T / dV^T
  static_assert(NC % 4 == 0, "copies must split over the four waves");
  // separate LDS objects per buffer, so that a copy in flight into one does
  // not hold up reads of another
  __shared__ __attribute__((aligned(1024))) uint8_t q_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t q_lds1[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t d_lds0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t d_lds1[TILE];
  __shared__ __attribute__((aligned(16))) float st_lds0[64];   // 32 LSE, 32 Delta
  __shared__ __attribute__((aligned(16))) float st_lds1[64];

  // work item: (kv head, 64-key block, sequence), kv head fastest, sequence
  // slowest; key block 0 (the most causal work) first
  const int lin = blockIdx.x;
  const int g = lin % a.num_kv_heads;
  const int rest = lin / a.num_kv_heads;
  const int kblk = rest % a.n_kblocks;
  const int b = rest / a.n_kblocks;
  int s0 = a.cu_seqlens[b];
  int s1 = a.cu_seqlens[b + 1];
  s0 = s0 < 0 ? 0 : (s0 > a.total_tokens ? a.total_tokens : s0);
  s1 = s1 < s0 ? s0 : (s1 > a.total_tokens ? a.total_tokens : s1);
  const int L = s1 - s0;
  const int kb0 = kblk * 4 * KW;
  if (kb0 >= L) return;   // uniform over the workgroup

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15, j4 = lane >> 4;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = a.group;
  const float c = a.c;
  const int kw0 = kb0 + KW * wave;                   // this wave's first key
  const int key = kw0 + c16;                         // this lane's key column
  const bool key_ok = key < L;
  const bool wave_live = kw0 < L;

  const uint32_t qaddr0 = (uint32_t)(uintptr_t)(MIATTN_LDS uint8_t*)q_lds0;
  const uint32_t qaddr1 = (uint32_t)(uintptr_t)(MIATTN_LDS uint8_t*)q_lds1;
  const uint32_t daddr0 = (uint32_t)(uintptr_t)(MIATTN_LDS uint8_t*)d_lds0;
  const uint32_t daddr1 = (uint32_t)(uintptr_t)(MIATTN_LDS uint8_t*)d_lds1;
  const uint32_t saddr0 = (uint32_t)(uintptr_t)(MIATTN_LDS float*)st_lds0;
  const uint32_t saddr1 = (uint32_t)(uintptr_t)(MIATTN_LDS float*)st_lds1;

  // K and V of this lane's key as B operands (fp16 copies): d = 32 ks + 8 j4
  // .. + 7; keys past the sequence end repeat its last key (masked below)
  u32x4 kreg[NKS], vreg[NKS];
  {
    const int kr = key_ok ? key : L - 1;
    const size_t off = ((size_t)(s0 + kr) * Hkv + g) * D + 8 * j4;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kreg[ks] = ld16(a.k16 + off + 32 * ks);
      vreg[ks] = ld16(a.v16 + off + 32 * ks);
    }
  }

  // steps: (query tile, query head of the group), the last query tile first
  // and the heads fastest, down to (causal) the tile holding query kb0; all
  // four waves take every step (the walk order shares L2 as above)
  const int n_qt = (L + QT - 1) / QT;
  const int qt0 = CAUSAL ? kb0 / QT : 0;
  const int nq = n_qt - qt0;
  const int n_steps = G * nq;

  // copy j of a tile (this wave's NCW of the NC): lane fills slot lidx % CH of
  // row lidx / CH (lidx = 64 j + lane) with the chunk the swizzle maps there;
  // rows past the sequence end repeat its last row (their P and dS are 0)
  const size_t q_row = (size_t)Hq * D;
  uint32_t qoff[NCW];
#pragma unroll
  for (int jj = 0; jj < NCW; ++jj) {
    const int lidx = (wave * NCW + jj) * 64 + lane;
    const int r = lidx / CH;
    const int slot = lidx % CH;
    qoff[jj] = (uint32_t)(((size_t)r * q_row + 8 * (slot ^ TL::swz(r))) * 2);
  }
  const uint32_t st_lane = (uint32_t)(((lane >= 8 ? (size_t)Hq * a.t_pad : 0) + 4 * (lane & 7)) * 4);
  auto load_tile = [&](int st, int buf) {
    const int h = g * G + st % G;
    const int q0 = (n_qt - 1 - st / G) * QT;
    const bool full = q0 + QT <= L;
    const char* qsrc = (const char*)(a.q16 + ((size_t)(s0 + q0) * Hq + h) * D);
    const char* dsrc = (const char*)(a.do16 + ((size_t)(s0 + q0) * Hq + h) * D);
#pragma unroll
    for (int jj = 0; jj < NCW; ++jj) {
      uint32_t off = qoff[jj];
      if (!full) {
        const int r = ((wave * NCW + jj) * 64 + lane) / CH;
        const int rr = q0 + r < L ? r : L - 1 - q0;
        off -= (uint32_t)((size_t)(r - rr) * q_row * 2);
      }
      const uint32_t lo = (uint32_t)((wave * NCW + jj) * 1024);
      dma16_to_lds_asm(qsrc, off, (buf ? qaddr1 : qaddr0) + lo);
      dma16_to_lds_asm(dsrc, off, (buf ? daddr1 : daddr0) + lo);
    }
    if (wave == 0 && lane < 16)
      dma16_to_lds_asm(a.stats, st_lane + (uint32_t)(((size_t)h * a.t_pad + s0 + q0) * 4), buf ? saddr1 : saddr0);
  };

  f32x4 dk_acc[NDB], dv_acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      dk_acc[i][r] = 0.f;
      dv_acc[i][r] = 0.f;
    }

  if (n_steps > 0) load_tile(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  for (int i = 0; i < n_steps; ++i) {
    const int buf = i & 1;
    if (i + 1 < n_steps) load_tile(i + 1, buf ^ 1);
    const int q0 = (n_qt - 1 - i / G) * QT;
    // a causal step whose queries all precede this wave's keys adds nothing
    if (wave_live && (!CAUSAL || q0 + QT - 1 >= kw0)) {
      const MIATTN_LDS uint8_t* ql = (const MIATTN_LDS uint8_t*)(uintptr_t)(buf ? qaddr1 : qaddr0);
      const MIATTN_LDS uint8_t* dl_ = (const MIATTN_LDS uint8_t*)(uintptr_t)(buf ? daddr1 : daddr0);
      const MIATTN_LDS float* sl = (const MIATTN_LDS float*)(uintptr_t)(buf ? saddr1 : saddr0);
      // S = Q K^T and dP = dO V^T for the two 16-query blocks: A = query row
      // 16 qb + c16, chunk 4 ks + j4
      f32x4 s[2], dp[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        s[qb] = (f32x4){0.f, 0.f, 0.f, 0.f};
        dp[qb] = (f32x4){0.f, 0.f, 0.f, 0.f};
        const int r = 16 * qb + c16;
        auto so = [&](int ks) { return r * (2 * D) + 16 * ((4 * ks + j4) ^ TL::swz(r)); };
        u32x4 oq = lds_ld16(ql + so(0)), od = lds_ld16(dl_ + so(0));
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          u32x4 nq_ = oq, nd = od;
          if (ks + 1 < NKS) {
            nq_ = lds_ld16(ql + so(ks + 1));
            nd = lds_ld16(dl_ + so(ks + 1));
          }
          s[qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(oq), as_f16x8(kreg[ks]), s[qb], 0, 0, 0);
          dp[qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(od), as_f16x8(vreg[ks]), dp[qb], 0, 0, 0);
          oq = nq_; od = nd;
        }
      }
      // this lane's rows 16 qb + 4 j4 + e: LSE (log2) and Delta
      float l2[2][4], dl[2][4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const f32x4 lv = *reinterpret_cast<const MIATTN_LDS f32x4*>(sl + 16 * qb + 4 * j4);
        const f32x4 dv = *reinterpret_cast<const MIATTN_LDS f32x4*>(sl + 32 + 16 * qb + 4 * j4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          l2[qb][e] = lv[e];
          dl[qb][e] = dv[e];
        }
      }
      // the mask on the exponential's inputs, on tail and diagonal steps only
      const bool need_mask = kw0 + KW > L || q0 + QT > L || (CAUSAL && kw0 + KW - 1 > q0);
      if (need_mask) {
        asm volatile("" ::: "memory");   // keep this a branch: the common step skips it
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int qrow = q0 + 16 * qb + 4 * j4 + e;
            const bool ok = key_ok & (qrow < L) & (!CAUSAL | (key <= qrow));
            s[qb][e] = ok ? s[qb][e] : kNegInf;
            l2[qb][e] = ok ? l2[qb][e] : 0.f;
            dl[qb][e] = ok ? dl[qb][e] : 0.f;
          }
      }
      u32x4 pw, dsw;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float p[4], d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] = exp2_hw(__builtin_fmaf(s[qb][e], c, -l2[qb][e]));
          d[e] = p[e] * (dp[qb][e] - dl[qb][e]);
        }
        pw[2 * qb] = pack_f16x2(p[0], p[1]);
        pw[2 * qb + 1] = pack_f16x2(p[2], p[3]);
        dsw[2 * qb] = pack_f16x2(d[0], d[1]);
        dsw[2 * qb + 1] = pack_f16x2(d[2], d[3]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS: block j4 of 16 lanes reads query
      // rows 4 j4 + {0..3} and 16 + 4 j4 + {0..3}, head-dim columns
      // 16 db + {0..15}, through the transposing read
      const int r0 = 4 * j4 + (c16 >> 2);
      const int r1 = r0 + 16;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int col = 16 * db + 4 * (c16 & 3);
        const int ch = col >> 3, sub = (col & 7) * 2;
        const int o0 = r0 * (2 * D) + 16 * (ch ^ TL::swz(r0)) + sub;
        const int o1 = r1 * (2 * D) + 16 * (ch ^ TL::swz(r1)) + sub;
        const f16x8 dot = as_f16x8(lds_ld_tr16(dl_ + o0), lds_ld_tr16(dl_ + o1));
        const f16x8 qtr = as_f16x8(lds_ld_tr16(ql + o0), lds_ld_tr16(ql + o1));
        dv_acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dot, as_f16x8(pw), dv_acc[db], 0, 0, 0);
        dk_acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qtr, as_f16x8(dsw), dk_acc[db], 0, 0, 0);
      }
    }
    // the next step's copies (every wave's) have landed, and no wave still
    // reads the buffer the step after will fill
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // lane: key kw0 + c16, head-dim columns 16 db + 4 j4 .. + 3 of block db
  if (key_ok) {
    const size_t go = ((size_t)(s0 + key) * Hkv + g) * D + 4 * j4;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const f32x4 kv = dk_acc[db] * sc;
      const f32x4 vv = dv_acc[db];
      u32x2 wk = {pack_bf16x2(kv[0], kv[1]), pack_bf16x2(kv[2], kv[3])};
      u32x2 wv = {pack_bf16x2(vv[0], vv[1]), pack_bf16x2(vv[2], vv[3])};
      *reinterpret_cast<u32x2*>(a.dk + go + 16 * db) = wk;
      *reinterpret_cast<u32x2*>(a.dv + go + 16 * db) = wv;
    }
  }
}

// ---------------------------------------------------------------- dQ
// Workgroup = 4 waves over NH (the largest of 4, 2, 1 dividing G) query heads of one kv head and 4/NH
// blocks of 32 query rows; K/V tiles of 32 KB keys are shared by the waves.
// At head_dim 256 (KB = 1) Q and dO as operands and dQ^T take 256 registers,
// so one workgroup runs per CU.
template <int D, int KB, bool CAUSAL>
__global__ __launch_bounds__(256, D >= 256 ? 1 : 2) void miattn_bwd_dq_kernel(BwdArgs a) {
  using TL = BwdTile<D>;
  constexpr int CH = TL::CH;
  constexpr int BC = 32 * KB;
  constexpr int NKK = D / 16;
  constexpr int NDT = D / 32;
  constexpr int TILE_BYTES = BC * D * 2;
  constexpr int NI = TILE_BYTES / 1024 / 4;
  static_assert(TILE_BYTES % 4096 == 0, "tile must split into 1-KB copies over 4 waves");
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[TILE_BYTES];
  auto kbuf = [&](int i) { return (MIATTN_LDS uint8_t*)(i == 0 ? k_lds0 : k_lds1); };
  auto vbuf = [&](int i) { return (MIATTN_LDS uint8_t*)(i == 0 ? v_lds0 : v_lds1); };

  const int NH = a.heads_per_wg;
  const int WQ = 4 / NH;
  const int QR = 32 * WQ;

  // work item: (head slot, query tile, sequence), head slot fastest, sequence
  // slowest (one sequence's K/V stays in L2); the last query tiles (the most
  // causal work) first
  const int lin = blockIdx.x;
  const int hslot = lin % a.n_head_slots;
  const int rest = lin / a.n_head_slots;
  const int unit = rest % a.n_qunits;
  const int b = rest / a.n_qunits;
  int s0 = a.cu_seqlens[b];
  int s1 = a.cu_seqlens[b + 1];
  s0 = s0 < 0 ? 0 : (s0 > a.total_tokens ? a.total_tokens : s0);
  s1 = s1 < s0 ? s0 : (s1 > a.total_tokens ? a.total_tokens : s1);
  const int L = s1 - s0;
  const int n_tiles = (L + QR - 1) / QR;
  if (unit >= n_tiles) return;   // uniform over the workgroup
  const int qt = n_tiles - 1 - unit;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int bb = lane >> 4, kq = lane & 15;
  const int hs = wave % NH;
  const int qs = wave / NH;
  const int gpw = a.group / NH;
  const int g = hslot / gpw;
  const int h = g * a.group + (hslot % gpw) * NH + hs;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const float c = a.c;
  const int q0 = qt * QR + 32 * qs;
  const int qrow = q0 + (lane & 31);
  const bool q_ok = qrow < L;

  // Q and dO of this lane's query row as B operands (fp16 copies); its LSE
  // and Delta
  u32x4 qop[NKK], dop[NKK];
  float l2, dlt;
  {
    const size_t off = ((size_t)(s0 + (q_ok ? qrow : 0)) * Hq + h) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      qop[kk] = q_ok ? ld16(a.q16 + off + 16 * kk) : z;
      dop[kk] = q_ok ? ld16(a.do16 + off + 16 * kk) : z;
    }
    const size_t si = (size_t)h * a.t_pad + s0 + (q_ok ? qrow : 0);
    l2 = a.stats[si];
    dlt = a.stats[(size_t)Hq * a.t_pad + si];
  }

  const size_t kv_row = (size_t)Hkv * D;
  const uint16_t* kbase = a.k16 + (size_t)s0 * kv_row + (size_t)g * D;
  const uint16_t* vbase = a.v16 + (size_t)s0 * kv_row + (size_t)g * D;
  uint32_t koff[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int lidx = (wave * NI + j) * 64 + lane;
    const int r = lidx / CH;
    const int slot = lidx % CH;
    koff[j] = (uint32_t)(((size_t)r * kv_row + 8 * (slot ^ TL::swz(r))) * 2);
  }
  const uint64_t tile_bytes = (uint64_t)BC * kv_row * 2;
  auto load_tile = [&](int kt, int buf) {
    const bool full = (kt + 1) * BC <= L;
    const char* kb0 = (const char*)kbase + (uint64_t)kt * tile_bytes;
    const char* vb0 = (const char*)vbase + (uint64_t)kt * tile_bytes;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      uint32_t off = koff[j];
      if (!full) {
        const int r = ((wave * NI + j) * 64 + lane) / CH;
        const int rr = kt * BC + r < L ? r : L - 1 - kt * BC;
        off -= (uint32_t)((size_t)(r - rr) * kv_row * 2);
      }
      dma16_to_lds(kb0, off, kbuf(buf) + (wave * NI + j) * 1024);
      dma16_to_lds(vb0, off, vbuf(buf) + (wave * NI + j) * 1024);
    }
  };

  const int kend_wg = CAUSAL ? (qt * QR + QR < L ? qt * QR + QR : L) : L;
  const int n_kt = (kend_wg + BC - 1) / BC;
  const int kend_w = CAUSAL ? (q0 + 32 < L ? q0 + 32 : L) : L;
  const int n_kt_w = q0 < L ? (kend_w + BC - 1) / BC : 0;

  f32x16 acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  if (n_kt > 0) load_tile(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  auto step = [&](int kt, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    if (kt + 1 < n_kt) load_tile(kt + 1, buf ^ 1);
    if (kt < n_kt_w) {
      const MIATTN_LDS uint8_t* kl = kbuf(buf);
      const MIATTN_LDS uint8_t* vl = vbuf(buf);
      const bool need_mask = (kt + 1) * BC > L || (CAUSAL && (kt + 1) * BC - 1 > q0);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        // S^T = K Q^T and dP^T = V dO^T: A = key row 32 kb + lane%32
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[r] = 0.f;
          dp[r] = 0.f;
        }
        const int r = 32 * kb + (lane & 31);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const int so = r * (2 * D) + 16 * ((2 * kk + half) ^ TL::swz(r));
          s = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(lds_ld16(kl + so)), as_f16x8(qop[kk]), s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(lds_ld16(vl + so)), as_f16x8(dop[kk]), dp, 0, 0, 0);
        }
        // dS^T = P^T (dP^T - Delta), 0 outside the sequence and above the
        // diagonal: on tail and diagonal tiles only, masked scores become
        // -inf (P = 0, dS = 0 * (dP - Delta) = 0; K/V rows past the end repeat
        // the last one, so dP stays finite). Key of element e: kt BC + 32 kb +
        // 4 half + (8 (e / 4) + e % 4), kept iff that offset is below lim.
        // Rows past the end (q_ok false) are computed and never written.
        if (need_mask) {
          asm volatile("" ::: "memory");   // keep this a branch: the common tile skips it
          const int kbase_lane = kt * BC + 32 * kb + 4 * half;
          int lim = L - kbase_lane;
          if (CAUSAL) {
            const int lc = qrow + 1 - kbase_lane;
            lim = lc < lim ? lc : lim;
          }
#pragma unroll
          for (int e = 0; e < 16; ++e) s[e] = (8 * (e >> 2) + (e & 3)) < lim ? s[e] : kNegInf;
        }
        u32x4 dsw[2];
#pragma unroll
        for (int e0 = 0; e0 < 16; e0 += 2) {
          float d[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int e = e0 + u;
            const float p = exp2_hw(__builtin_fmaf(s[e], c, -l2));
            d[u] = p * (dp[e] - dlt);
          }
          dsw[e0 >> 3][(e0 >> 1) & 3] = pack_f16x2(d[0], d[1]);
        }
        // dQ^T += K^T dS^T; K^T rows (keys) through the transposing read
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r0 = 32 * kb + 16 * u + 4 * (bb >> 1) + (kq >> 2);
          const int r1 = r0 + 8;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const int col = 32 * dt + 16 * (bb & 1) + 4 * (kq & 3);
            const int ch = col >> 3, sub = (col & 7) * 2;
            const f16x8 ktr = as_f16x8(lds_ld_tr16(kl + r0 * (2 * D) + 16 * (ch ^ TL::swz(r0)) + sub),
                                       lds_ld_tr16(kl + r1 * (2 * D) + 16 * (ch ^ TL::swz(r1)) + sub));
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ktr, as_f16x8(dsw[u]), acc[dt], 0, 0, 0);
          }
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  for (int kt = 0; kt < n_kt; kt += 2) {
    step(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < n_kt) step(kt + 1, std::integral_constant<int, 1>{});
  }

  if (q_ok) {
    uint16_t* qp = a.dq + ((size_t)(s0 + qrow) * Hq + h) * D + 4 * half;
    const float sc = a.scale;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x16& A = acc[dt];
        u32x2 w = {pack_bf16x2(A[4 * r4] * sc, A[4 * r4 + 1] * sc), pack_bf16x2(A[4 * r4 + 2] * sc, A[4 * r4 + 3] * sc)};
        *reinterpret_cast<u32x2*>(qp + 32 * dt + 8 * r4) = w;
      }
  }
}

}  // namespace miattn
