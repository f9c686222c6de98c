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
//  * delta: Delta = rowsum(dO * O) in fp32, one pass over O and dO.
//  * dK/dV: one workgroup of 4 waves per (kv head, 128 keys, sequence); each
//    wave keeps its 32 keys' K and V as MFMA operands in registers and its
//    dK^T, dV^T in accumulators, while tiles of 32 queries of Q and dO (for
//    every query head of the group, so GQA sums stay in registers) stream
//    through LDS by direct HBM->LDS copies, double-buffered. Per tile:
//    S = Q K^T and dP = dO V^T (query rows, key columns), then
//    dV^T += dO^T P and dK^T += Q^T dS: the accumulator registers of P and dS,
//    rounded to fp16, are the B operand as they stand; dO^T and Q^T come from
//    the same LDS tile through the transposing read.
//  * dQ: the forward's orientation: one wave per 32 query rows of one head,
//    S^T = K Q^T and dP^T = V dO^T with Q, dO held as operands, K/V tiles
//    streaming through LDS, dQ^T += K^T dS^T with K^T read transposed.
// dQ is not accumulated inside the dK/dV kernel, which would need atomics or
// an ordering between workgroups: the dQ kernel recomputes S and dP instead
// (7 products per key/query pair instead of 5).
// Operands are fp16, not bf16: each lane converts the 16 bytes its own direct
// copy wrote once the copy has landed (before the barrier that publishes the
// tile), and register operands once at the start. The bf16 inputs convert
// exactly (inside fp16's range); P and dS are then rounded to fp16 (11
// significant bits) instead of bf16 (8) for the three gradient products. The
// gradients are unbounded sums of such products, and with bf16 P and dS their
// error alone exceeds the bf16 output bar for magnitudes above ~2.
#pragma once
#include <type_traits>

#include "common.h"

namespace miattn {

struct BwdArgs {
  const uint16_t* q;          // [T, Hq, D]
  const uint16_t* k;          // [T, Hkv, D]
  const uint16_t* v;
  const uint16_t* o;          // [T, Hq, D] forward output
  const uint16_t* dout;       // [T, Hq, D]
  const float* lse;           // [Hq, T] forward log-sum-exp (natural log)
  float* delta;               // [Hq, T] workspace
  uint16_t* dq;               // [T, Hq, D]
  uint16_t* dk;               // [T, Hkv, D]
  uint16_t* dv;
  const int32_t* cu_seqlens;  // [num_seqs + 1]
  int num_seqs;
  int total_tokens;
  int num_q_heads;
  int num_kv_heads;
  int group;                  // G
  int heads_per_wg;           // dQ kernel: query heads per workgroup (NH)
  int n_units;                // grid units per sequence (key blocks or query tiles)
  int n_head_slots;           // dQ kernel: Hkv * G / NH
  float c;                    // scale * log2(e)
  float scale;
};

// LDS tile of R rows x D bf16 read both ways: as a 128-bit operand (16
// consecutive rows x one 16-byte chunk per cycle) and through the transposing
// read (4 consecutive rows x 4 consecutive chunks per cycle). Chunk c of row
// r sits in slot c ^ swz(r). D >= 128 (16+ slots per row, one row per 64
// banks): swz = 4 (r mod 4) + (r / 4) mod 4 gives 16 consecutive rows 16
// different slots, and 4 consecutive rows 4 different groups of 4 slots.
// D = 64 (two rows per 64 banks): the same on r / 2, with the parity of r
// choosing the half of the banks.
template <int D>
struct BwdTile {
  static constexpr int CH = D / 8;
  __device__ static int swz(int r) {
    return CH >= 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
};

// ---------------------------------------------------------------- delta
// One row (token, head) per CH = D/8 lanes; 16-byte loads of O and dO, fp32
// products, an xor-tree over the CH lanes.
template <int D>
__global__ __launch_bounds__(256) void miattn_bwd_delta_kernel(BwdArgs a) {
  constexpr int CH = D / 8;
  constexpr int RPB = 256 / CH;
  const int t = threadIdx.x;
  const long row = (long)blockIdx.x * RPB + t / CH;   // token * Hq + head
  const long rows = (long)a.total_tokens * a.num_q_heads;
  const int ch = t % CH;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 ov = ld16(a.o + row * D + 8 * ch);
    const u32x4 dv = ld16(a.dout + row * D + 8 * ch);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += bf16lo_to_f32(ov[i]) * bf16lo_to_f32(dv[i]);
      acc += bf16hi_to_f32(ov[i]) * bf16hi_to_f32(dv[i]);
    }
  }
#pragma unroll
  for (int m = CH / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, CH);
  if (row < rows && ch == 0) {
    const long tok = row / a.num_q_heads;
    const int h = (int)(row % a.num_q_heads);
    a.delta[(size_t)h * a.total_tokens + tok] = acc;
  }
}

// Forward log-sum-exp in log2 units of the raw score times c; a row that saw
// no key (-inf) gives +inf, i.e. P = 0.
__device__ __forceinline__ float lse_to_log2(float lse) {
  return lse == kNegInf ? __builtin_inff() : lse * kLog2e;
}

// ---------------------------------------------------------------- dK / dV
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void miattn_bwd_dkdv_kernel(BwdArgs a) {
  using TL = BwdTile<D>;
  constexpr int CH = TL::CH;
  constexpr int NKK = D / 16;                        // MFMA steps over the head dim
  constexpr int NDT = D / 32;                        // 32-wide d blocks of dK^T / dV^T
  constexpr int QT = 32;                             // queries per tile
  constexpr int TILE_BYTES = QT * D * 2;
  constexpr int NI = TILE_BYTES / 1024 / 4;          // 1-KB copies per wave per tensor
  static_assert(TILE_BYTES % 4096 == 0, "tile must split into 1-KB copies over 4 waves");
  __shared__ __attribute__((aligned(1024))) uint8_t q_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t q_lds1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t d_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t d_lds1[TILE_BYTES];
  auto qbuf = [&](int i) { return (MIATTN_LDS uint8_t*)(i == 0 ? q_lds0 : q_lds1); };
  auto dbuf = [&](int i) { return (MIATTN_LDS uint8_t*)(i == 0 ? d_lds0 : d_lds1); };

  // work item: (kv head, key block, sequence), kv head fastest; key block 0
  // (the most causal work) first
  const int lin = blockIdx.x;
  const int g = lin % a.num_kv_heads;
  const int rest = lin / a.num_kv_heads;
  const int kblk = rest / a.num_seqs;
  const int b = rest % a.num_seqs;
  int s0 = a.cu_seqlens[b];
  int s1 = a.cu_seqlens[b + 1];
  s0 = s0 < 0 ? 0 : (s0 > a.total_tokens ? a.total_tokens : s0);
  s1 = s1 < s0 ? s0 : (s1 > a.total_tokens ? a.total_tokens : s1);
  const int L = s1 - s0;
  const int kb0 = kblk * 128;
  if (kb0 >= L) return;   // uniform over the workgroup

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int bb = lane >> 4, kq = lane & 15;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads, G = a.group;
  const float c = a.c;
  const int key = kb0 + 32 * wave + (lane & 31);     // this lane's key column
  const bool key_ok = key < L;

  // K, V of the wave's 32 keys as B operands: lane holds key lane%32,
  // d = 16 kk + 8 half + 0..7
  u32x4 kop[NKK], vop[NKK];
  {
    const size_t off = ((size_t)(s0 + (key_ok ? key : 0)) * Hkv + g) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      kop[kk] = key_ok ? bf16x8_to_f16x8(ld16(a.k + off + 16 * kk)) : z;
      vop[kk] = key_ok ? bf16x8_to_f16x8(ld16(a.v + off + 16 * kk)) : z;
    }
  }

  // query tiles: causal tiles start at the one holding query kb0
  const int n_qt = (L + QT - 1) / QT;
  const int qt0 = CAUSAL ? kb0 / QT : 0;
  const int nq = n_qt - qt0;
  const int n_steps = G * nq;

  // copies of tile (head h, query tile qt): lane i of copy j fills slot
  // lidx % CH of row lidx / CH with the chunk the swizzle maps there; rows
  // past the sequence end repeat its last row (their P is masked to 0)
  const size_t q_row = (size_t)Hq * D;
  uint32_t qoff[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int lidx = (wave * NI + j) * 64 + lane;
    const int r = lidx / CH;
    const int slot = lidx % CH;
    qoff[j] = (uint32_t)(((size_t)r * q_row + 8 * (slot ^ TL::swz(r))) * 2);
  }
  auto step_head = [&](int st) { return g * G + st / nq; };
  auto step_tile = [&](int st) { return qt0 + st % nq; };
  auto load_tile = [&](int st, int buf) {
    const int h = step_head(st);
    const int q0 = step_tile(st) * QT;
    const bool full = q0 + QT <= L;
    const char* qb0 = (const char*)(a.q + ((size_t)(s0 + q0) * Hq + h) * D);
    const char* db0 = (const char*)(a.dout + ((size_t)(s0 + q0) * Hq + h) * D);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      uint32_t off = qoff[j];
      if (!full) {
        const int r = ((wave * NI + j) * 64 + lane) / CH;
        const int rr = q0 + r < L ? r : L - 1 - q0;
        off -= (uint32_t)((size_t)(r - rr) * q_row * 2);
      }
      dma16_to_lds(qb0, off, qbuf(buf) + (wave * NI + j) * 1024);
      dma16_to_lds(db0, off, dbuf(buf) + (wave * NI + j) * 1024);
    }
  };
  // bf16 -> fp16 in place, on the 16 bytes this lane's copies wrote; the
  // copies must have landed (vmcnt(0)), the barrier after publishes the tile
  auto convert_own = [&](int buf) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      MIATTN_LDS uint8_t* pq = qbuf(buf) + (wave * NI + j) * 1024 + 16 * lane;
      MIATTN_LDS uint8_t* pd = dbuf(buf) + (wave * NI + j) * 1024 + 16 * lane;
      lds_st16(pq, bf16x8_to_f16x8(lds_ld16(pq)));
      lds_st16(pd, bf16x8_to_f16x8(lds_ld16(pd)));
    }
  };
  // log2-unit LSE and Delta of the 16 query rows a lane's S elements belong
  // to: rows 8 (i/4) + 4 half + i%4 of the tile
  auto load_stats = [&](int st, float* l2, float* dl) {
    const int h = step_head(st);
    const int q0 = step_tile(st) * QT;
    const float* lp = a.lse + (size_t)h * a.total_tokens + s0;
    const float* dp = a.delta + (size_t)h * a.total_tokens + s0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int row = q0 + 8 * (i >> 2) + 4 * half + (i & 3);
      row = row < L ? row : L - 1;
      l2[i] = lse_to_log2(lp[row]);
      dl[i] = dp[row];
    }
  };

  f32x16 dk_acc[NDT], dv_acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk_acc[i][r] = 0.f;
      dv_acc[i][r] = 0.f;
    }

  float l2[16], dl[16];
  if (n_steps > 0) {
    load_tile(0, 0);
    load_stats(0, l2, dl);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (n_steps > 0) convert_own(0);
  __syncthreads();

  auto step = [&](int st, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    if (st + 1 < n_steps) load_tile(st + 1, buf ^ 1);
    const MIATTN_LDS uint8_t* ql = qbuf(buf);
    const MIATTN_LDS uint8_t* dl_ = dbuf(buf);
    const int q0 = step_tile(st) * QT;
    // S = Q K^T and dP = dO V^T: A = row lane%32 of the tile, chunk 2 kk + half
    f32x16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = 0.f;
      dp[r] = 0.f;
    }
    {
      const int r = lane & 31;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int so = r * (2 * D) + 16 * ((2 * kk + half) ^ TL::swz(r));
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(lds_ld16(ql + so)), as_f16x8(kop[kk]), s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(lds_ld16(dl_ + so)), as_f16x8(vop[kk]), dp, 0, 0, 0);
      }
    }
    // P = exp2(s c - lse2) and dS = P (dP - Delta), masked to 0 outside the
    // sequence and (causal) above the diagonal
    u32x4 pw[2], dsw[2];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      float p[2], d[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int qrow = q0 + 8 * ((i + e) >> 2) + 4 * half + ((i + e) & 3);
        const bool ok = key_ok && qrow < L && (!CAUSAL || key <= qrow);
        p[e] = ok ? exp2_hw(__builtin_fmaf(s[i + e], c, -l2[i + e])) : 0.f;
        d[e] = p[e] * (dp[i + e] - dl[i + e]);
      }
      pw[i >> 3][(i >> 1) & 3] = pack_f16x2(p[0], p[1]);
      dsw[i >> 3][(i >> 1) & 3] = pack_f16x2(d[0], d[1]);
    }
    if (st + 1 < n_steps) load_stats(st + 1, l2, dl);
    // dV^T += dO^T P and dK^T += Q^T dS; X^T rows through the transposing
    // read: block bb of 16 lanes reads rows 16u + 4(bb/2) + {0..3} (+8),
    // columns 32 dt + 16 (bb%2) + {0..15}
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r0 = 16 * u + 4 * (bb >> 1) + (kq >> 2);
      const int r1 = r0 + 8;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int col = 32 * dt + 16 * (bb & 1) + 4 * (kq & 3);
        const int ch = col >> 3, sub = (col & 7) * 2;
        const int o0 = r0 * (2 * D) + 16 * (ch ^ TL::swz(r0)) + sub;
        const int o1 = r1 * (2 * D) + 16 * (ch ^ TL::swz(r1)) + sub;
        const f16x8 dot = as_f16x8(lds_ld_tr16(dl_ + o0), lds_ld_tr16(dl_ + o1));
        const f16x8 qtr = as_f16x8(lds_ld_tr16(ql + o0), lds_ld_tr16(ql + o1));
        dv_acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(dot, as_f16x8(pw[u]), dv_acc[dt], 0, 0, 0);
        dk_acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(qtr, as_f16x8(dsw[u]), dk_acc[dt], 0, 0, 0);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // tile st+1 has landed in LDS
    if (st + 1 < n_steps) convert_own(buf ^ 1);
    __syncthreads();
  };
  for (int st = 0; st < n_steps; st += 2) {
    step(st, std::integral_constant<int, 0>{});
    if (st + 1 < n_steps) step(st + 1, std::integral_constant<int, 1>{});
  }

  // epilogue: lane holds key lane%32, d = 32 dt + 8 r4 + 4 half + 0..3
  if (key_ok) {
    uint16_t* kp = a.dk + ((size_t)(s0 + key) * Hkv + g) * D + 4 * half;
    uint16_t* vp = a.dv + ((size_t)(s0 + key) * Hkv + g) * D + 4 * half;
    const float sc = a.scale;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x16& K = dk_acc[dt];
        const f32x16& V = dv_acc[dt];
        u32x2 wk = {pack_bf16x2(K[4 * r4] * sc, K[4 * r4 + 1] * sc), pack_bf16x2(K[4 * r4 + 2] * sc, K[4 * r4 + 3] * sc)};
        u32x2 wv = {pack_bf16x2(V[4 * r4], V[4 * r4 + 1]), pack_bf16x2(V[4 * r4 + 2], V[4 * r4 + 3])};
        *reinterpret_cast<u32x2*>(kp + 32 * dt + 8 * r4) = wk;
        *reinterpret_cast<u32x2*>(vp + 32 * dt + 8 * r4) = wv;
      }
  }
}

// ---------------------------------------------------------------- dQ
// Workgroup = 4 waves over NH = min(G, 4) query heads of one kv head and 4/NH
// blocks of 32 query rows; K/V tiles of 32 KB keys are shared by the waves.
template <int D, int KB, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void miattn_bwd_dq_kernel(BwdArgs a) {
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

  // work item: (head slot, query tile, sequence), head slot fastest; the last
  // query tiles (the most causal work) first
  const int lin = blockIdx.x;
  const int hslot = lin % a.n_head_slots;
  const int rest = lin / a.n_head_slots;
  const int b = rest % a.num_seqs;
  const int unit = rest / a.num_seqs;
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

  // Q and dO of this lane's query row as B operands; its LSE and Delta
  u32x4 qop[NKK], dop[NKK];
  float l2, dlt;
  {
    const size_t off = ((size_t)(s0 + (q_ok ? qrow : 0)) * Hq + h) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      qop[kk] = q_ok ? bf16x8_to_f16x8(ld16(a.q + off + 16 * kk)) : z;
      dop[kk] = q_ok ? bf16x8_to_f16x8(ld16(a.dout + off + 16 * kk)) : z;
    }
    const size_t si = (size_t)h * a.total_tokens + s0 + (q_ok ? qrow : 0);
    l2 = lse_to_log2(a.lse[si]);
    dlt = a.delta[si];
  }

  const size_t kv_row = (size_t)Hkv * D;
  const uint16_t* kbase = a.k + (size_t)s0 * kv_row + (size_t)g * D;
  const uint16_t* vbase = a.v + (size_t)s0 * kv_row + (size_t)g * D;
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
  auto convert_own = [&](int buf) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      MIATTN_LDS uint8_t* pk = kbuf(buf) + (wave * NI + j) * 1024 + 16 * lane;
      MIATTN_LDS uint8_t* pv = vbuf(buf) + (wave * NI + j) * 1024 + 16 * lane;
      lds_st16(pk, bf16x8_to_f16x8(lds_ld16(pk)));
      lds_st16(pv, bf16x8_to_f16x8(lds_ld16(pv)));
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
  if (n_kt > 0) convert_own(0);
  __syncthreads();

  auto step = [&](int kt, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    if (kt + 1 < n_kt) load_tile(kt + 1, buf ^ 1);
    if (kt < n_kt_w) {
      const MIATTN_LDS uint8_t* kl = kbuf(buf);
      const MIATTN_LDS uint8_t* vl = vbuf(buf);
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
        // dS^T = P^T (dP^T - Delta), masked outside the sequence and above
        // the diagonal
        u32x4 dsw[2];
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          float d[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int key = kt * BC + 32 * kb + 8 * ((i + e) >> 2) + 4 * half + ((i + e) & 3);
            const bool ok = q_ok && key < L && (!CAUSAL || key <= qrow);
            const float p = ok ? exp2_hw(__builtin_fmaf(s[i + e], c, -l2)) : 0.f;
            d[e] = p * (dp[i + e] - dlt);
          }
          dsw[i >> 3][(i >> 1) & 3] = pack_f16x2(d[0], d[1]);
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
    if (kt + 1 < n_kt) convert_own(buf ^ 1);
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
