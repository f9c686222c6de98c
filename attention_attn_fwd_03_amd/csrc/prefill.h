// Tiled prefill forward with an online softmax on gfx950 (bf16 MFMA).
//
// The loop is the FlashAttention forward of "Streaming process" (steps 3-8
// and its code snippet): Q is loaded once, K/V tiles stream through on-chip
// memory while the previous tile is consumed, S = Q K^T lands in fp32
// registers, the row max / exponentials / rescaling run on the vector ALUs,
// P V accumulates into registers, and O / l is cast to bf16 at the end.
//
// MI355X mapping:
//  * Workgroup = 4 waves. Waves split the NH query heads of one kv-head group
//    (NH = min(G, 4)) and 4/NH blocks of 32 query rows, so every wave reuses
//    the same K/V tile from LDS (GQA sharing of "GPU Datapath", section C).
//  * K/V tiles of Bc = 32*KB keys are double-buffered in LDS. The next tile is
//    fetched into registers with coalesced 16-byte loads while the current
//    tile is consumed, then written to the other LDS buffer; one barrier per
//    tile.
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
//  * Grid: one workgroup per (kv-head group, query tile, sequence), with the
//    head index varying fastest (workgroups are dealt to the 8 XCDs round
//    robin, so a kv head's K/V stays in one XCD's L2 when there are 8 of
//    them) and the query tiles in decreasing order (heaviest causal tiles
//    first).
#pragma once
#include <type_traits>

#include "common.h"

namespace miattn {

struct FwdArgs {
  const uint16_t* q;          // [T, Hq, D]
  const uint16_t* k;          // [T, Hkv, D]
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
  int n_qtiles;               // query tiles per sequence (ceil(max_seqlen / QR))
  int n_head_slots;           // Hkv * G / NH
  float c;                    // scale * log2(e)
};

constexpr float kFwdRescaleThreshold = 8.0f;

template <int D, int KB>
struct FwdSmem {
  static constexpr int BC = 32 * KB;
  static constexpr int KROW = D + 8;     // bf16 elements per K row in LDS (16-B pad)
  static constexpr int VROW = D + 32;    // bf16 elements per V row in LDS (64-B pad)
  static constexpr int KBYTES = BC * KROW * 2;
  static constexpr int VBYTES = BC * VROW * 2;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int BYTES = 2 * STAGE;
  static constexpr int CHUNKS = BC * D / 8;          // 16-byte chunks per K (or V) tile
  static constexpr int PER_THREAD = CHUNKS / 256;
  static_assert(CHUNKS % 256 == 0, "tile must split evenly over 256 threads");
};

template <int D, int KB, bool CAUSAL>
__global__ __launch_bounds__(256, D >= 256 ? 1 : 2) void miattn_prefill_fwd_kernel(FwdArgs a) {
  using SM = FwdSmem<D, KB>;
  constexpr int BC = SM::BC;
  constexpr int NKK = D / 16;   // MFMA steps over the head dim (16 each)
  constexpr int NDT = D / 32;   // 32-wide output column tiles
  __shared__ __attribute__((aligned(16))) uint8_t smem[SM::BYTES];

  const int NH = a.heads_per_wg;
  const int WQ = 4 / NH;
  const int QR = 32 * WQ;

  // --- work item ---------------------------------------------------------
  const int lin = blockIdx.x;
  const int hslot = lin % a.n_head_slots;
  const int rest = lin / a.n_head_slots;
  const int qt = a.n_qtiles - 1 - rest / a.num_seqs;
  const int b = rest % a.num_seqs;
  int s0 = a.cu_seqlens[b];
  int s1 = a.cu_seqlens[b + 1];
  s0 = s0 < 0 ? 0 : (s0 > a.total_tokens ? a.total_tokens : s0);
  s1 = s1 < s0 ? s0 : (s1 > a.total_tokens ? a.total_tokens : s1);
  const int L = s1 - s0;
  const int q0 = qt * QR;
  if (q0 >= L) return;   // uniform over the workgroup

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hs = wave % NH;
  const int qs = wave / NH;
  const int gpw = a.group / NH;                 // workgroups per kv head
  const int g = hslot / gpw;
  const int h = g * a.group + (hslot % gpw) * NH + hs;
  const int qrow = q0 + 32 * qs + (lane & 31);  // this lane's query position
  const int half = lane >> 5;                   // 0/1: which 16 of each 32 keys
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;

  // --- Q operand (B of S^T = K Q^T): row qrow, d = 16kk + 8 half .. +7 ------
  u32x4 qop[NKK];
  {
    const bool ok = qrow < L;
    const uint16_t* qp = a.q + ((size_t)(s0 + (ok ? qrow : 0)) * Hq + h) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 z = {0u, 0u, 0u, 0u};
      qop[kk] = ok ? ld16(qp + 16 * kk) : z;
    }
  }

  // --- KV extent --------------------------------------------------------
  const int kend_wg = CAUSAL ? (L < q0 + QR ? L : q0 + QR) : L;
  const int n_kt = (kend_wg + BC - 1) / BC;
  const int wq_lo = q0 + 32 * qs;                // first query row of this wave
  const int kend_w = CAUSAL ? (L < wq_lo + 32 ? L : wq_lo + 32) : L;
  const int n_kt_w = (kend_w + BC - 1) / BC;     // tiles this wave needs

  const size_t kv_row = (size_t)Hkv * D;
  const uint16_t* kbase = a.k + (size_t)s0 * kv_row + (size_t)g * D;
  const uint16_t* vbase = a.v + (size_t)s0 * kv_row + (size_t)g * D;

  u32x4 kreg[SM::PER_THREAD], vreg[SM::PER_THREAD];
  // Global -> registers for tile kt. Rows past the sequence end (tail tile
  // only) read the last valid row and are then zeroed, so the loads never
  // branch and nothing outside the sequence reaches P.V.
  auto fetch = [&](int kt) {
    const bool full = (kt + 1) * BC <= L;
#pragma unroll
    for (int it = 0; it < SM::PER_THREAD; ++it) {
      const int id = it * 256 + threadIdx.x;
      const int r = id / (D / 8);
      const int c8 = (id % (D / 8)) * 8;
      const int key = kt * BC + r;
      const int krow = full ? key : (key < L ? key : L - 1);
      const size_t off = (size_t)krow * kv_row + c8;
      kreg[it] = ld16(kbase + off);
      vreg[it] = ld16(vbase + off);
    }
    if (!full) {
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int it = 0; it < SM::PER_THREAD; ++it) {
        const int id = it * 256 + threadIdx.x;
        const bool bad = kt * BC + id / (D / 8) >= L;
        kreg[it] = bad ? z : kreg[it];
        vreg[it] = bad ? z : vreg[it];
      }
    }
  };
  auto stash = [&](int buf) {
    MIATTN_LDS uint16_t* kl = (MIATTN_LDS uint16_t*)(smem + buf * SM::STAGE);
    MIATTN_LDS uint16_t* vl = (MIATTN_LDS uint16_t*)(smem + buf * SM::STAGE + SM::KBYTES);
#pragma unroll
    for (int it = 0; it < SM::PER_THREAD; ++it) {
      const int id = it * 256 + threadIdx.x;
      const int r = id / (D / 8);
      const int c8 = (id % (D / 8)) * 8;
      lds_st16(kl + r * SM::KROW + c8, kreg[it]);
      lds_st16(vl + r * SM::VROW + c8, vreg[it]);
    }
  };

  float m = kNegInf;   // running max of this lane's query row (log2 units)
  float l = 0.f;       // running sum over the keys this lane holds
  f32x16 acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  const float c = a.c;
  const int bb = lane >> 4, kq = lane & 15;
  // per-lane LDS offsets (elements) of the K operand rows and the V^T reads
  const int k_off = (lane & 31) * SM::KROW + 8 * half;
  const int v_off = (4 * (bb >> 1) + (kq >> 2)) * SM::VROW + 16 * (bb & 1) + 4 * (kq & 3);

  // One K/V tile: S^T = K Q^T, online softmax, O^T += V^T P^T.
  auto tile = [&](int kt, int buf, bool need_mask) {
    const MIATTN_LDS uint16_t* kl = (const MIATTN_LDS uint16_t*)(smem + buf * SM::STAGE) + k_off;
    const MIATTN_LDS uint16_t* vl = (const MIATTN_LDS uint16_t*)(smem + buf * SM::STAGE + SM::KBYTES) + v_off;
    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(lds_ld16(kl + 32 * kb * SM::KROW + 16 * kk)), as_bf16x8(qop[kk]), s[kb], 0, 0, 0);
    }
    if (need_mask) {   // diagonal or tail tile only (uniform branch)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * BC + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool ok = key < L && (!CAUSAL || key <= qrow);
          s[kb][r] = ok ? s[kb][r] : kNegInf;
        }
    }
    // raw-score row max (scale > 0, so max(s * c) = c * max(s))
    float smax = kNegInf;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) smax = fmaxf(smax, s[kb][r]);
    smax = fmaxf(smax, xor32(smax));
    const float tmax = smax * c;
    if (__builtin_amdgcn_ballot_w64(tmax > m + kFwdRescaleThreshold)) {
      const float mn = fmaxf(m, tmax);
      const float alpha = (m == kNegInf) ? 0.f : exp2_hw(m - mn);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
      m = mn;
    }
    const float nmu = (m == kNegInf) ? 0.f : -m;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      uint32_t pw[8];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = exp2_hw(__builtin_fmaf(s[kb][r], c, nmu));
        const float p1 = exp2_hw(__builtin_fmaf(s[kb][r + 1], c, nmu));
        l += p0 + p1;
        pw[r >> 1] = pack_bf16x2(p0, p1);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32x4 pu = {pw[4 * u], pw[4 * u + 1], pw[4 * u + 2], pw[4 * u + 3]};
        const bf16x8 pop = as_bf16x8(pu);
        // V^T rows: keys 32kb + 16u + 4(lane/32) + {0..3} and the same + 8
        const MIATTN_LDS uint16_t* vp = vl + (32 * kb + 16 * u) * SM::VROW;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const u32x2 lo = lds_ld_tr16(vp + 32 * dt);
          const u32x2 hi = lds_ld_tr16(vp + 8 * SM::VROW + 32 * dt);
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lo, hi), pop, acc[dt], 0, 0, 0);
        }
      }
    }
  };

  fetch(0);
  stash(0);
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) fetch(kt + 1);
    if (kt < n_kt_w) {
      tile(kt, buf, (kt + 1) * BC > L || (CAUSAL && (kt + 1) * BC - 1 > wq_lo));
    }
    if (kt + 1 < n_kt) stash(buf ^ 1);
    __syncthreads();
  }

  // --- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 ----------------------
  l += xor32(l);
  if (qrow < L) {
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
    uint16_t* op = a.o + ((size_t)(s0 + qrow) * Hq + h) * D + 4 * half;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x16& A = acc[dt];
        u32x2 w = {pack_bf16x2(A[4 * r4] * inv, A[4 * r4 + 1] * inv),
                   pack_bf16x2(A[4 * r4 + 2] * inv, A[4 * r4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + 32 * dt + 8 * r4) = w;
      }
    if (a.lse != nullptr && half == 0)
      a.lse[(size_t)h * a.total_tokens + s0 + qrow] = empty ? kNegInf : (m + log2_hw(l)) * kLn2;
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

template <bool CAUSAL>
__global__ __launch_bounds__(64) void miattn_prefill_fwd_f32_kernel(FwdF32Args a) {
  constexpr int D = 64;
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
  if (q0 >= L) return;
  const int lane = threadIdx.x;
  const int half = lane >> 5;
  const int qrow = q0 + (lane & 31);
  const int g = h / a.group;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const size_t kv_row = (size_t)Hkv * D;

  // Q operand: lane holds d = 2 st + half for st = 0..31
  float qv[32];
  {
    const bool ok = qrow < L;
    const float* qp = a.q + ((size_t)(s0 + (ok ? qrow : 0)) * Hq + h) * D + half;
#pragma unroll
    for (int st = 0; st < 32; ++st) qv[st] = ok ? qp[2 * st] : 0.f;
  }
  const int kend = CAUSAL ? (L < q0 + 32 ? L : q0 + 32) : L;
  float m = kNegInf, l = 0.f;
  f32x16 acc[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) { acc[0][r] = 0.f; acc[1][r] = 0.f; }
  const float* kb = a.k + (size_t)s0 * kv_row + (size_t)g * D;
  const float* vb = a.v + (size_t)s0 * kv_row + (size_t)g * D;

  for (int k0 = 0; k0 < kend; k0 += 32) {
    // S^T (32 keys x 32 queries); A = K (row key k0 + lane%32, col d = 2 st + half)
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    const int krow = k0 + (lane & 31);
    const bool kok = krow < L;
    const float* kp = kb + (size_t)(kok ? krow : 0) * kv_row + half;
#pragma unroll
    for (int st = 0; st < 32; ++st)
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(kok ? kp[2 * st] : 0.f, qv[st], s, 0, 0, 0);
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
    // O^T += V^T P^T, step r pairs key 8(r/4) + r%4 (lanes < 32) with key + 4
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + 8 * (r >> 2) + 4 * half + (r & 3);
      const bool ok = key < L;
      const float* vp = vb + (size_t)(ok ? key : 0) * kv_row + (lane & 31);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(ok ? vp[32 * dt] : 0.f, s[r], acc[dt], 0, 0, 0);
    }
  }
  l += xor32(l);
  if (qrow < L) {
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
    float* op = a.o + ((size_t)(s0 + qrow) * Hq + h) * D + 4 * half;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 w = {acc[dt][4 * r4] * inv, acc[dt][4 * r4 + 1] * inv, acc[dt][4 * r4 + 2] * inv,
                   acc[dt][4 * r4 + 3] * inv};
        *reinterpret_cast<f32x4*>(op + 32 * dt + 8 * r4) = w;
      }
    if (a.lse != nullptr && half == 0)
      a.lse[(size_t)h * a.total_tokens + s0 + qrow] = empty ? kNegInf : (m + log2_hw(l)) * kLn2;
  }
}

}  // namespace miattn
