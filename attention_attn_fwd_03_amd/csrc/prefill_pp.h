// Tiled prefill forward, ping-pong form (dense K/V, head_dim 64 and 128;
// causal, and non-causal as the causal code with every key visible).
//
// The same computation as miattn_prefill_fwd_kernel (the FlashAttention
// forward of "Streaming process", steps 3-8: S = Q K^T per K/V tile, online
// softmax, O += P V, O / l at the end), scheduled so that the matrix cores
// and the vector ALUs of every SIMD work at the same time.
//
// A workgroup holds 8 waves, two groups of four; waves w and w + 4 run on the
// same SIMD, so each SIMD carries one wave of each group. Work per K/V tile t
// splits into two phases:
//   GEMM(t): O += P(t-1) V(t-1) and S(t) = K(t) Q^T   (32 MFMAs for D = 128)
//   SOFT(t): mask, exponentials, P(t) in bf16          (vector ALU only)
// Group 1 runs one phase behind group 0: with one workgroup barrier per
// tile, interval t holds GEMM(t), SOFT(t) for group 0 and SOFT(t - 1),
// GEMM(t) for group 1, so one wave of each SIMD issues MFMAs while the other
// computes exponentials, first one way round, then the other. Both groups
// walk the same program order; only their barriers sit at different points.
//
// Every wave of interval t reads K(t) and V(t - 1). At the start of interval
// u each wave starts its share of the direct HBM->LDS copies of K(u + 1) and
// V(u) into the buffers that K(u - 1) and V(u - 2) held (read last in
// interval u - 1, closed by the barrier) and waits for them at the end of
// interval u, before the barrier, so both tiles are in LDS when interval
// u + 1 reads them. Two buffers each for K and V. A
// workgroup takes two query tiles in turn; the second tile's Q rows are
// loaded in the first one's last step (its last S is done, no copy is in
// flight), so their latency hides behind the last P V and the epilogue.
// The epilogue stages each wave's normalised output in the (then free) K/V
// buffers and writes whole rows, 16 bytes per lane: a direct store from the
// accumulator layout would write 8 bytes into each of 32 rows per instruction.
//
// Lanes, swizzles and MFMA shapes follow the four-wave kernel: S^T = K Q^T on
// 32x32x16 bf16 MFMAs (lane l owns query row l % 32, 16 of every 32 keys),
// V^T through ds_read_b64_tr_b16, the lazy running max (moves only when a
// tile's max exceeds it by more than 2^8; the tile max is taken only when the
// tile's probabilities against the current max could reach that). Tiles,
// accumulation orders and the softmax rule are the four-wave kernel's, so
// both give the same bits.
#pragma once

#include "prefill.h"

namespace miattn {

// Scheduling template for NM MFMAs fed from LDS: AHEAD reads first, then
// each MFMA followed by the NDS reads of a later one, so operand reads run a
// few MFMAs ahead without holding every operand of the phase in registers.
template <int NM, int NDS, int AHEAD>
__device__ __forceinline__ void pp_mfma_reads() {
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);   // LDS reads
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);    // LDS reads
  }
}

template <int D, int KB, bool CAUSAL, bool F16V = false>
__global__ __launch_bounds__(512, 1) void miattn_prefill_pp_kernel(FwdArgs a) {
  constexpr int BC = 32 * KB;   // keys per tile
  using TL = FwdTile<D, KB>;
  constexpr int CH = TL::CH;
  constexpr int NKK = D / 16;
  constexpr int NDT = D / 32;
  constexpr int NI = TL::TILE_BYTES / 1024 / 8;   // 1-KB copies per wave per tensor and tile
  static_assert(TL::TILE_BYTES % 8192 == 0, "tile must split into 1-KB copies over 8 waves");
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[TL::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[TL::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[TL::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[TL::TILE_BYTES];
  auto kbuf = [&](int i) { return (MIATTN_LDS uint8_t*)(i == 0 ? k_lds0 : k_lds1); };
  auto vbuf = [&](int i) { return (MIATTN_LDS uint8_t*)(i == 0 ? v_lds0 : v_lds1); };
  auto lds_addr = [&](MIATTN_LDS uint8_t* p) { return (uint32_t)(uintptr_t)p; };

  const int NH = a.heads_per_wg;
  const int WQ = 4 / NH;
  const int QR = 64 * WQ;   // query rows per tile: two groups of WQ 32-row blocks

  // --- work item: (head slot, tile pair, sequence); head slot fastest ------
  const int lin = blockIdx.x;
  const int hslot = lin % a.n_head_slots;
  const int rest = lin / a.n_head_slots;
  // sequence-major: the workgroups resident together read one sequence's
  // K/V, which then stays in L2
  const int pair = rest % a.n_pairs;
  const int b = rest / a.n_pairs;
  int s0 = a.cu_seqlens[b];
  int s1 = a.cu_seqlens[b + 1];
  s0 = s0 < 0 ? 0 : (s0 > a.total_tokens ? a.total_tokens : s0);
  s1 = s1 < s0 ? s0 : (s1 > a.total_tokens ? a.total_tokens : s1);
  const int Lq = s1 - s0;
  const int Lk = Lq;
  // query i sees keys j <= i + off: 0 for causal; Lk (every key visible)
  // for non-causal, which then runs the same code with only the tail tile
  // masked. The non-causal value is made opaque to the compiler: folded into
  // a separate non-causal form, the kernel ran short of scalar registers and
  // lost its operand prefetch.
  int off = 0;
  if (!CAUSAL) {
    off = Lk;
    asm volatile("" : "+s"(off));
  }
  const int n_tiles = (Lq + QR - 1) / QR;
  // query tiles i and n-1-i together cost the same for every pair (causal)
  if (pair > n_tiles - 1 - pair) return;   // uniform over the workgroup
  const int n_mine = pair != n_tiles - 1 - pair ? 2 : 1;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2;       // ping-pong group
  const int w4 = wave & 3;
  const int hs = w4 % NH;
  const int qs = w4 / NH;
  const int gpw = a.group / NH;
  const int g = hslot / gpw;
  const int h = g * a.group + (hslot % gpw) * NH + hs;
  const int half = lane >> 5;
  const int Hq = a.num_q_heads;
  const int Hkv = a.num_kv_heads;
  const float c = a.c;

  const size_t kv_row = (size_t)Hkv * D;
  const uint16_t* kbase = a.k + (size_t)s0 * kv_row + (size_t)g * D;
  const uint16_t* vbase = a.v + (size_t)s0 * kv_row + (size_t)g * D;

  // Direct global -> LDS copies: lane i of copy j of this wave fills slot
  // lidx % CH of row lidx / CH, lidx = (wave NI + j) 64 + i, with the chunk
  // the swizzle maps there. Rows past the last key repeat it (their scores
  // are masked, their probabilities 0).
  uint32_t koff[NI], voff[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int lidx = (wave * NI + j) * 64 + lane;
    const int r = lidx / CH;
    const int slot = lidx % CH;
    const size_t rowpart = (size_t)r * kv_row;
    koff[j] = (uint32_t)((rowpart + 8 * (slot ^ TL::kswz(r))) * 2);
    voff[j] = (uint32_t)((rowpart + 8 * (slot ^ TL::vswz(r))) * 2);
  }
  const uint64_t tile_bytes = (uint64_t)BC * kv_row * 2;
  // copies of tile kt of one tensor (base: K or V, offs: its lane offsets)
  // dst: LDS byte address of the buffer. The copies are not tracked by the
  // compiler; the phase loop waits for them before the barrier that
  // publishes them.
  auto copy_tile = [&](int kt, const uint16_t* base, const uint32_t* offs, uint32_t dst)
      __attribute__((always_inline)) {
    const bool full = (kt + 1) * BC <= Lk;
    const char* b0 = (const char*)base + (uint64_t)kt * tile_bytes;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      uint32_t o = offs[j];
      if (!full) {
        const int r = ((wave * NI + j) * 64 + lane) / CH;
        const int rr = kt * BC + r < Lk ? r : Lk - 1 - kt * BC;
        o -= (uint32_t)((size_t)(r - rr) * kv_row * 2);
      }
      dma16_to_lds_asm(b0, o, dst + (wave * NI + j) * 1024);
    }
  };

  const int bb = lane >> 4, kq = lane & 15;
  // LDS operand addresses, as a per-lane part plus a per-lane XOR term plus
  // compile-time offsets (block and half-tile rows fold into instruction
  // immediates). K: row 32 kb + lr, chunk (2 kk + half) ^ kswz(lr); the
  // swizzle depends on lr only, and chunk * 16 = 32 (kk ^ (sw >> 1)) +
  // 16 (half ^ (sw & 1)). V^T: row r0 = 32 kb + 16 u + rl (and r0 + 8), chunk
  // (4 dt + c0) ^ vswz(rl), with vswz a multiple of 4 that depends on rl only.
  const int lr = lane & 31;
  const int ksw = TL::kswz(lr);
  const uint32_t k_lane = (uint32_t)(lr * (2 * D) + 16 * (half ^ (ksw & 1)));
  const uint32_t k_x = (uint32_t)((ksw >> 1) << 5);
  const int rl = 4 * (bb >> 1) + (kq >> 2);
  const int c0 = 2 * (bb & 1) + ((kq & 3) >> 1);
  const uint32_t v_lane = (uint32_t)(rl * (2 * D) + 16 * c0 + 8 * (kq & 1));
  const uint32_t v_x = (uint32_t)((TL::vswz(rl) >> 2) << 6);

  auto tile_of = [&](int ts) { return ts == 0 ? pair : n_tiles - 1 - pair; };
  // Q rows of this wave for query tile qt, straight into B-operand registers
  // (rows past the last query as zeros)
  u32x4 qop[NKK];
  auto load_q = [&](int qt) __attribute__((always_inline)) {
    const int row = qt * QR + 32 * (grp * WQ + qs) + (lane & 31);
    const bool ok = row < Lq;
    const uint16_t* qp = a.q + ((size_t)(s0 + (ok ? row : 0)) * Hq + h) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      qop[kk] = ok ? ld16(qp + 16 * kk) : z;
    }
  };
  load_q(tile_of(0));

  for (int tsel = 0; tsel < n_mine; ++tsel) {
    const int qt = tile_of(tsel);
    const int q0 = qt * QR + 32 * (grp * WQ + qs);   // first query row of this wave

    auto clampk = [&](int x) { return x < 0 ? 0 : (x > Lk ? Lk : x); };
    const int kend_wg = clampk(qt * QR + QR + off);
    const int n_kt = (kend_wg + BC - 1) / BC;   // tiles of the workgroup
    const int kend_w = clampk(q0 + 32 + off);
    const int n_kt_w = q0 < Lq ? (kend_w + BC - 1) / BC : 0;   // tiles this wave computes

    float m = kNegInf, l = 0.f;
    f32x16 acc[NDT];
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    f32x16 s[KB];
    u32x4 pw[KB][2];

    if (tsel > 0) __syncthreads();   // the previous tile's last reads are done
    if (n_kt > 0) copy_tile(0, kbase, koff, lds_addr(kbuf(0)));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // The Q rows have landed (the wait above covers every load). Reading
    // their registers here lets the compiler see that: otherwise it places
    // its own vmcnt waits before the loop's first score products, where they
    // would also wait for the K/V copies issued for the next tile.
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) asm volatile("" ::"v"(qop[kk]));
    __syncthreads();

    // GEMM(t): P(t-1) V(t-1) into O (pv), then S(t) = K(t) Q^T (qk)
    auto pv = [&](int t) __attribute__((always_inline)) {
      if (t >= 1 && t - 1 < n_kt_w) {
        const MIATTN_LDS uint8_t* vl = vbuf((t - 1) & 1) + v_lane;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
              const MIATTN_LDS uint8_t* vp = vl + (((uint32_t)(64 * dt)) ^ v_x) + (32 * kb + 16 * u) * (2 * D);
              const u32x2 lo = lds_ld_tr16(vp);
              const u32x2 hi = lds_ld_tr16(vp + 8 * (2 * D));
              acc[dt] = mfma_pv<F16V>(lo, hi, pw[kb][u], acc[dt]);
            }
          }
        pp_mfma_reads<KB * 2 * NDT, 2, 8>();
      }
    };
    auto qk = [&](int t) __attribute__((always_inline)) {
      if (t < n_kt_w) {
        const MIATTN_LDS uint8_t* kl = kbuf(t & 1) + k_lane;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const bf16x8 kop = as_bf16x8(lds_ld16(kl + (((uint32_t)(32 * kk)) ^ k_x) + 32 * kb * (2 * D)));
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, as_bf16x8(qop[kk]), s[kb], 0, 0, 0);
          }
        pp_mfma_reads<NKK * KB, 1, 4>();
      }
    };
    // SOFT(t): mask, lazy rescale, P(t) = exp2(s c - m) in bf16
    auto soft = [&](int t) __attribute__((always_inline)) {
      if (t >= n_kt_w) return;
      const bool need_mask = (t + 1) * BC > Lk || (t + 1) * BC - 1 > q0 + off;
      if (need_mask) {
        // key of score r in block kb: t BC + 4 half + (32 kb + 8 (r / 4) + r % 4);
        // it is kept iff that offset is below lim (one compare with an
        // immediate per score, no per-score registers)
        const int kbase_lane = t * BC + 4 * half;
        int lim = Lk - kbase_lane;
        const int lc = q0 + (lane & 31) + off + 1 - kbase_lane;
        lim = lc < lim ? lc : lim;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[kb][r] = (32 * kb + 8 * (r >> 2) + (r & 3)) < lim ? s[kb][r] : kNegInf;
      }
      // P(t) = exp2(s c - m) in bf16 and the tile's row sum ls (fp32 values,
      // summed in score order, then added to l)
      // (the sum starts from the first pair: the probabilities are never
      // negative, so this is the bits of 0 + ..., one add fewer)
      auto exps = [&](float nmu) __attribute__((always_inline)) {
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const float p0 = exp2_hw(__builtin_fmaf(s[kb][r], c, nmu));
            const float p1 = exp2_hw(__builtin_fmaf(s[kb][r + 1], c, nmu));
            ls = (kb == 0 && r == 0) ? p0 + p1 : ls + (p0 + p1);
            pw[kb][r >> 3][(r >> 1) & 3] = pack_p<F16V>(p0, p1);
          }
        return ls;
      };
      // The running max moves only when the tile's max exceeds it by more
      // than 2^8 (the four-wave kernel's rule, whose bits this kernel
      // reproduces). That needs the tile max only when some probability
      // taken against the current max could exceed 2^8: with a finite max in
      // every lane and every lane's sum at most 2^6, no score is within 2
      // (log2 units) of the threshold, so the rule keeps the max and the
      // probabilities already computed are the ones it would give. Otherwise
      // (the first tile, a large or non-finite sum) take the max and apply
      // the rule, then recompute.
      bool slow = __builtin_amdgcn_ballot_w64(m == kNegInf) != 0;
      float ls = 0.f;
      if (!slow) {
        ls = exps(-m);
        slow = __builtin_amdgcn_ballot_w64(!(ls <= 64.f)) != 0;
      }
      if (slow) {
        float smax = kNegInf;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) smax = fmaxf(smax, s[kb][r]);
        smax = fmaxf(smax, xor32(smax));
        const float tmax = smax * c;   // scale > 0, so max(s c) = c max(s)
        if (__builtin_amdgcn_ballot_w64(tmax > m + kFwdRescaleThreshold)) {
          const float mn = fmaxf(m, tmax);
          const float alpha = (m == kNegInf) ? 0.f : exp2_hw(m - mn);
          l *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
          m = mn;
        }
        ls = exps((m == kNegInf) ? 0.f : -m);
      }
      l += ls;
    };

    // Both groups walk the same sequence GEMM(i), SOFT(i) in program order,
    // so the accumulators keep one register home (two orders, one per group,
    // made the compiler copy them between homes and spill).
    auto copies = [&](int u) __attribute__((always_inline)) {
      if (u + 1 < n_kt) copy_tile(u + 1, kbase, koff, lds_addr(kbuf((u + 1) & 1)));
      if (u < n_kt) copy_tile(u, vbase, voff, lds_addr(vbuf(u & 1)));
    };
    // One barrier per tile: interval i is GEMM(i), SOFT(i) for group 0 and
    // SOFT(i - 1), GEMM(i) for group 1 (the same program order, the barriers
    // at different points); every wave of interval i reads K(i) and V(i - 1),
    // and each wave issues its share of the copies of K(i + 1) and V(i) right
    // after the barrier that opens the interval and waits for it at its end.
    // The last interval (i = n_kt) holds only P(n_kt - 1) V(n_kt - 1); no
    // copy is in flight and Q is dead (the last S was in interval n_kt - 1):
    // the next query tile's Q rows are loaded there and travel through the
    // last P V and the epilogue; the next pass's first wait covers them. That
    // interval sits outside the loop, so no Q load is pending inside it.
    if (grp == 1) copies(0);
    for (int i = 0; i < n_kt; ++i) {
      if (grp == 0) copies(i);
      // the wave in its MFMA half of the interval issues first when both
      // waves of a SIMD have an instruction ready
      __builtin_amdgcn_s_setprio(1);
      pv(i);
      qk(i);
      __builtin_amdgcn_s_setprio(0);
      if (grp == 1) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        copies(i + 1);
      }
      soft(i);
      if (grp == 0) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
      }
    }
    if (tsel + 1 < n_mine) load_q(tile_of(tsel + 1));
    __builtin_amdgcn_s_setprio(1);
    pv(n_kt);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();

    // --- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 --------------------
    // After the loop's last barrier the K/V buffers are free: each wave stages
    // its 32 x D block of O there (bf16, chunk c of row r in slot c ^ (r mod
    // CH, at most 16)), then stores whole rows, 16 bytes per lane.
    const float lt = l + xor32(l);
    const int qrow = q0 + (lane & 31);
    const bool empty = !(lt > 0.f);
    const float inv = empty ? 0.f : 1.f / lt;
    constexpr int OB = 32 * D * 2;   // bytes of one wave's block
    static_assert(2 * OB <= TL::TILE_BYTES, "two waves' blocks per K/V buffer");
    auto osw = [&](int r) { return r & (CH >= 16 ? 15 : CH - 1); };
    MIATTN_LDS uint8_t* stg = ((wave >> 2) ? vbuf((wave >> 1) & 1) : kbuf((wave >> 1) & 1)) + (wave & 1) * OB;
    {
      const int r = lane & 31;
      MIATTN_LDS uint8_t* sr = stg + r * (2 * D) + 8 * half;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x16& A = acc[dt];
          u32x2 w = {pack_bf16x2(A[4 * r4] * inv, A[4 * r4 + 1] * inv),
                     pack_bf16x2(A[4 * r4 + 2] * inv, A[4 * r4 + 3] * inv)};
          *reinterpret_cast<MIATTN_LDS u32x2*>(sr + 16 * ((4 * dt + r4) ^ osw(r))) = w;
        }
    }
    // the lane index from an opaque instruction, so that the store addresses
    // are formed here rather than held through the loop
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
#pragma unroll
    for (int j = 0; j < 32 * CH / 64; ++j) {
      const int lidx = 64 * j + ln;
      const int r = lidx / CH, ch = lidx % CH;
      const u32x4 w = lds_ld16(stg + r * (2 * D) + 16 * (ch ^ osw(r)));
      if (q0 + r < Lq) st16_stream(a.o + ((size_t)(s0 + q0 + r) * Hq + h) * D + 8 * ch, w);
    }
    if (qrow < Lq && a.lse != nullptr && half == 0)
      a.lse[(size_t)h * a.total_tokens + s0 + qrow] = empty ? kNegInf : (m + log2_hw(lt)) * kLn2;
  }
}

}  // namespace miattn
