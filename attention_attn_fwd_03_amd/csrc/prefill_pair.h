// Dense prefill at head_dim 256 on pairs of specialised waves (gfx950, bf16
// Q/K, fp16 V).
//
// At head_dim 256 a wave that owns 32 query rows and does all of their work
// holds their output (32 x 256 fp32: 128 registers) and their Q rows as
// operands (64), so the four-wave kernel runs one wave per SIMD and nothing
// hides its latencies. Here two waves on one SIMD share each block of 32
// query rows and split the loop of "Streaming process" (steps 3-8) by role:
//  * the score wave holds the Q rows and computes S^T = K Q^T for key tile t
//    (16 MFMAs of 32x32x16 over the head dim), which it stores in LDS;
//  * the output wave holds O, the running max and sum: it takes tile t - 1's
//    scores from LDS, masks them, applies the lazy rescale, forms P and
//    accumulates O^T += V^T P^T (16 MFMAs).
// Phase k of the loop runs the score wave on the k-th key tile of the walk
// and the output wave on the one before, with a workgroup barrier after each
// phase, so on every SIMD one wave's exponentials overlap the other's
// matrix-core work. Both waves fit two per SIMD (about 110 and 180
// registers). The copies of the next phase's K tile and this phase's V tile
// into LDS are issued in phase k (K and V tiles double-buffered, the score
// exchange too). Each work item is one query tile, the heaviest first; its
// key tiles are walked downwards from the diagonal. The grid is persistent
// and draws items from per-XCD work queues (see the work-item note below).
// Scores, softmax rule and roundings are those of the four-wave kernel
// (prefill.h); the online softmax visits the key tiles in the other order,
// which changes the result only by rounding. P.V runs on fp16 operands: V is
// converted to fp16 beforehand and the probabilities are rounded to fp16.
#pragma once
#include <type_traits>

#include "common.h"
#include "prefill.h"

namespace miattn {

template <bool CAUSAL>
__global__ __launch_bounds__(512, 1) void miattn_prefill_pair_kernel(FwdArgs a) {
  constexpr int D = 256;
  constexpr int BC = 32;         // keys per tile
  constexpr int CH = D / 8;      // 16-byte chunks per row
  constexpr int TILE_BYTES = BC * D * 2;
  constexpr int NI = TILE_BYTES / 1024 / 8;   // 1-KB copies per wave per tensor
  constexpr int NKK = D / 16;    // MFMA steps over the head dim
  constexpr int NDT = D / 32;    // 32-wide output column tiles
  using TL = FwdTile<D, 1>;
  static_assert(TILE_BYTES % 8192 == 0, "tile must split into 1-KB copies over 8 waves");
  // distinct LDS objects per buffer, so a copy in flight into one does not
  // hold up reads of another
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) f32x4 xs0[4][4][64];   // scores: [pair][quad][lane]
  __shared__ __attribute__((aligned(16))) f32x4 xs1[4][4][64];
  auto kbuf = [&](int i) { return (MIATTN_LDS uint8_t*)(i == 0 ? k_lds0 : k_lds1); };
  auto vbuf = [&](int i) { return (MIATTN_LDS uint8_t*)(i == 0 ? v_lds0 : v_lds1); };
  auto xbuf = [&](int i) { return (MIATTN_LDS f32x4*)(i == 0 ? &xs0[0][0][0] : &xs1[0][0][0]); };

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w4 = wave & 3;               // the row block: waves w4 and w4 + 4 share a SIMD
  const bool score_wave = wave < 4;

  // --- work items: (head slot, query tile, sequence); head slot fastest ----
  // One query tile per item, the heaviest (causal: the last) first, and all
  // tiles of one sequence before the next: the workgroups working together
  // on an XCD then walk the same key tiles at the same time, so one kv
  // head's K/V is read from L2 by all of them (causal pairs of tiles put
  // them at different key positions, and the K/V of a long sequence, 7.5 MB
  // per head at 7K tokens, does not fit an XCD's L2).
  //
  // The grid is persistent (one workgroup per compute unit) and takes items
  // from a work queue in device memory: item i belongs to queue i mod 8, and
  // a workgroup draws from the queue of the XCD it runs on (XCC_ID), so each
  // XCD serves the same items, in the same order, as when workgroup i of a
  // full grid was dealt to XCD i mod 8. An XCD whose queue is exhausted
  // draws from the others, so XCDs that run at a higher clock take more
  // items instead of waiting for the slowest. Each queue is one counter,
  // advanced with system-scope atomics so that the XCDs, each with its own
  // L2, act on one copy of it; a score wave draws the next item when its
  // loop ends, while the output waves write the current item's output.
  // Counters only grow, so every workgroup leaves once all queues are
  // exhausted; the last one to leave zeroes them for the next launch (calls
  // ordered on one stream share the counters, calls on other streams may not).
  unsigned* const wq = a.queue;
  int q_done = 0;   // (thread 0) queues, in visiting order, known to be exhausted
  auto grab = [&]() -> int {   // thread 0 only; -1 when every queue is exhausted
    const int n_items = a.n_head_slots * a.num_seqs * a.n_pairs;
    const int xcc = (int)__builtin_amdgcn_s_getreg(((4 - 1) << 11) | 20) & 7;   // hwreg(XCC_ID, 0, 4)
#pragma nounroll
    for (; q_done < 8; ++q_done) {
      const int y = (xcc + q_done) & 7;
      const int n_y = (n_items - y + 7) >> 3;   // items y, y + 8, ...
      if (n_y <= 0) continue;
      const int t = (int)__hip_atomic_fetch_add(wq + y, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      if (t < n_y) return 8 * t + y;
    }
    return -1;
  };
  __shared__ int item_slot[2];
  if (threadIdx.x == 0) item_slot[0] = grab();
  __syncthreads();

  for (int it = 0;; ++it) {
    const int lin = __builtin_amdgcn_readfirstlane(item_slot[it & 1]);
    if (lin < 0) break;
    // The arguments, read again for every item through an opaque pointer to
    // the kernel-argument segment: held through the item loop, they and the
    // values derived from them took more scalar registers than the kernel
    // has, and the spills changed the schedule of the inner loops.
    using KArgs = const __attribute__((address_space(4))) FwdArgs;
    KArgs* kp = (KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(kp));
    KArgs& a = *kp;   // shadows the parameter inside the item
    const int NH = a.heads_per_wg;
    const int WQ = 4 / NH;
    const int QR = 32 * WQ;   // query rows per tile
    const int hs = w4 % NH;
    const int qs = w4 / NH;
    const int gpw = a.group / NH;
    const int Hq = a.num_q_heads;
    const int Hkv = a.num_kv_heads;
    const float c = a.c;
    const size_t kv_row = (size_t)Hkv * D;
    const uint64_t tile_bytes = (uint64_t)BC * kv_row * 2;
    const int hslot = lin % a.n_head_slots;
    const int rest = lin / a.n_head_slots;
    const int unit = rest % a.n_pairs;
    const int b = rest / a.n_pairs;
    int s0 = a.cu_seqlens[b];
    int s1 = a.cu_seqlens[b + 1];
    s0 = s0 < 0 ? 0 : (s0 > a.total_tokens ? a.total_tokens : s0);
    s1 = s1 < s0 ? s0 : (s1 > a.total_tokens ? a.total_tokens : s1);
    const int L = s1 - s0;
    const int n_tiles = (L + QR - 1) / QR;
    int next = -1;   // (thread 0) the item after this one
    if (unit >= n_tiles) {
      // an empty slot: every later slot of this sequence is empty too, so
      // this queue moves past them at once
      if (threadIdx.x == 0) {
        const int y = lin & 7;
        const int lin_next = (b + 1) * a.n_pairs * a.n_head_slots;
        __hip_atomic_fetch_max(wq + y, (unsigned)((lin_next - y + 7) >> 3), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
        next = grab();
      }
    } else {
      // The lane index, made opaque anew for every item (its range stated
      // again), so that no lane-derived address is hoisted out of the item
      // loop: held across items, they pushed the kernel past its register
      // budget.
      int lane = threadIdx.x & 63;
      asm volatile("" : "+v"(lane));
      __builtin_assume(lane >= 0 && lane < 64);
      const int half = lane >> 5;
      // Direct global -> LDS copies of a K or V tile: lane i of copy j of
      // this wave fills slot lidx % CH of row lidx / CH (lidx = (wave NI + j)
      // 64 + i) with the chunk the swizzle maps there; rows past the
      // sequence end repeat its last row (their scores are masked).
      uint32_t koff[NI], voff[NI];
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int lidx = (wave * NI + j) * 64 + lane;
        const int r = lidx / CH;
        const int slot = lidx % CH;
        koff[j] = (uint32_t)(((size_t)r * kv_row + 8 * (slot ^ TL::kswz(r))) * 2);
        voff[j] = (uint32_t)(((size_t)r * kv_row + 8 * (slot ^ TL::vswz(r))) * 2);
      }
      const int bb = lane >> 4, kq = lane & 15;
      const int r_k = lane & 31;   // K row this lane reads as the A operand
      const int qt = n_tiles - 1 - unit;
      const int g = hslot / gpw;
      const int h = g * a.group + (hslot % gpw) * NH + hs;
      const uint16_t* kbase = a.k + (size_t)s0 * kv_row + (size_t)g * D;
      const uint16_t* vbase = a.v + (size_t)s0 * kv_row + (size_t)g * D;
      auto back_off = [&](int kt, int j) -> uint32_t {   // tail tile: rows past the end repeat the last one
        const int r = ((wave * NI + j) * 64 + lane) / CH;
        const int rr = kt * BC + r < L ? r : L - 1 - kt * BC;
        return (uint32_t)((size_t)(r - rr) * kv_row * 2);
      };
      auto load_k = [&](int kt, int buf) {
        const bool full = (kt + 1) * BC <= L;
        const char* b0 = (const char*)kbase + (uint64_t)kt * tile_bytes;
#pragma unroll
        for (int j = 0; j < NI; ++j)
          dma16_to_lds(b0, koff[j] - (full ? 0u : back_off(kt, j)), kbuf(buf) + (wave * NI + j) * 1024);
      };
      auto load_v = [&](int kt, int buf) {
        const bool full = (kt + 1) * BC <= L;
        const char* b0 = (const char*)vbase + (uint64_t)kt * tile_bytes;
#pragma unroll
        for (int j = 0; j < NI; ++j)
          dma16_to_lds(b0, voff[j] - (full ? 0u : back_off(kt, j)), vbuf(buf) + (wave * NI + j) * 1024);
      };

      const int q0 = qt * QR + 32 * qs;   // first query row of this block
      const int qt_end = qt * QR + QR;
      const int kend_wg = CAUSAL ? (qt_end < L ? qt_end : L) : L;
      const int n_kt = (kend_wg + BC - 1) / BC;
      const int kend_w = CAUSAL ? (q0 + 32 < L ? q0 + 32 : L) : L;
      const int n_kt_w = q0 < L ? (kend_w + BC - 1) / BC : 0;   // tiles this block computes
      // Key tiles are walked downwards, from the workgroup's last (the causal
      // diagonal, or the tail) to 0: with the heaviest tiles dealt first, the
      // workgroups resident on an XCD then move down one sequence's keys
      // together, a few tiles apart, and share them in L2. A block's first
      // tile always holds a key it sees. Phase k covers tile(k).
      auto tile = [&](int k) { return n_kt - 1 - k; };

      // The two roles run separate loops (so neither keeps the other's
      // registers live) with the same barriers: one or two before phase 0,
      // one after each of the n_kt + 1 phases. Phase k: the score wave on tile
      // k (K buffer k & 1, scores into exchange buffer k & 1), the output wave
      // on tile k - 1; every wave issues its share of the copies of K(k + 1)
      // and V(k).
      if (score_wave) {
        // Q rows as B operands: row q0 + lane%32, columns 16 kk + 8 half .. + 7
        u32x4 qop[NKK];
        {
          const int row = q0 + (lane & 31);
          const bool ok = row < L;
          const uint16_t* qp = a.q + ((size_t)(s0 + (ok ? row : 0)) * Hq + h) * D + 8 * half;
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            qop[kk] = ok ? ld16(qp + 16 * kk) : z;
          }
        }
        if (n_kt > 0) load_k(tile(0), 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        auto phase = [&](int k, auto parc) {
          constexpr int par = decltype(parc)::value;   // k & 1
          if (k + 1 < n_kt) load_k(tile(k + 1), par ^ 1);
          if (k < n_kt) load_v(tile(k), par);
          if (k < n_kt && tile(k) < n_kt_w) {
            f32x16 s;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = 0.f;
            const MIATTN_LDS uint8_t* kr = kbuf(par) + r_k * (2 * D);
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
              const bf16x8 kop = as_bf16x8(lds_ld16(kr + 16 * ((2 * kk + half) ^ TL::kswz(r_k))));
              s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, as_bf16x8(qop[kk]), s, 0, 0, 0);
            }
            MIATTN_LDS f32x4* xo = xbuf(par) + w4 * 256;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
              xo[r4 * 64 + lane] = (f32x4){s[4 * r4], s[4 * r4 + 1], s[4 * r4 + 2], s[4 * r4 + 3]};
          }
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
        };
        for (int k = 0; k <= n_kt; k += 2) {
          phase(k, std::integral_constant<int, 0>{});
          if (k + 1 <= n_kt) phase(k + 1, std::integral_constant<int, 1>{});
        }
        // draw the next item while the output waves write this one's output
        if (threadIdx.x == 0) next = grab();
      } else {
        float m = kNegInf, l = 0.f;
        f32x16 acc[NDT];
#pragma unroll
        for (int i = 0; i < NDT; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
        if (n_kt > 0) load_k(tile(0), 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        auto phase = [&](int k, auto parc) {
          constexpr int par = decltype(parc)::value;   // k & 1
          if (k + 1 < n_kt) load_k(tile(k + 1), par ^ 1);
          if (k < n_kt) load_v(tile(k), par);
          const int kt = tile(k - 1);   // the score wave's tile of the previous phase
          if (k >= 1 && kt < n_kt_w) {
            const MIATTN_LDS f32x4* xi = xbuf(par ^ 1) + w4 * 256;
            f32x16 s;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const f32x4 o = xi[r4 * 64 + lane];
#pragma unroll
              for (int e = 0; e < 4; ++e) s[4 * r4 + e] = o[e];
            }
            // mask (diagonal / tail tiles only): key of score r is kt BC +
            // 4 half + 8 (r / 4) + r % 4, kept iff that offset is below lim
            const bool need_mask = (kt + 1) * BC > L || (CAUSAL && (kt + 1) * BC - 1 > q0);
            if (need_mask) {
              const int kbase_lane = kt * BC + 4 * half;
              int lim = L - kbase_lane;
              if (CAUSAL) {
                const int lc = q0 + (lane & 31) + 1 - kbase_lane;
                lim = lc < lim ? lc : lim;
              }
#pragma unroll
              for (int r = 0; r < 16; ++r) s[r] = (8 * (r >> 2) + (r & 3)) < lim ? s[r] : kNegInf;
            }
            // tile max and lazy rescale (the running max moves only when the
            // tile's max exceeds it by more than 2^8)
            float smax = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) smax = fmaxf(smax, s[r]);
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
            // P = exp2(s c - m), rounded to fp16 for P.V; the tile's row sum
            // adds the fp32 values in score order, then l += ls
            const float nmu = (m == kNegInf) ? 0.f : -m;
            float ls = 0.f;
            u32x4 pw[2];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
              const float p0 = exp2_hw(__builtin_fmaf(s[r], c, nmu));
              const float p1 = exp2_hw(__builtin_fmaf(s[r + 1], c, nmu));
              ls += p0 + p1;
              pw[r >> 3][(r >> 1) & 3] = pack_f16x2(p0, p1);
            }
            // O^T += V^T P^T; V^T rows via the transposing read: block bb of
            // 16 lanes reads keys 16u + 4(bb/2) + {0..3} (+8), columns 32 dt +
            // 16 (bb%2) + {0..15}
            const MIATTN_LDS uint8_t* vl = vbuf(par ^ 1);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int r0 = 16 * u + 4 * (bb >> 1) + (kq >> 2);
              const int r1 = r0 + 8;
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt) {
                const int col = 32 * dt + 16 * (bb & 1) + 4 * (kq & 3);
                const int ch = col >> 3, sub = (col & 7) * 2;
                const u32x2 lo = lds_ld_tr16(vl + r0 * (2 * D) + 16 * (ch ^ TL::vswz(r0)) + sub);
                const u32x2 hi = lds_ld_tr16(vl + r1 * (2 * D) + 16 * (ch ^ TL::vswz(r1)) + sub);
                acc[dt] = mfma_pv<true>(lo, hi, pw[u], acc[dt]);
              }
            }
            l += ls;
          }
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
        };
        for (int k = 0; k <= n_kt; k += 2) {
          phase(k, std::integral_constant<int, 0>{});
          if (k + 1 <= n_kt) phase(k + 1, std::integral_constant<int, 1>{});
        }

        // --- epilogue: O = acc / l, LSE = (m + log2 l) ln 2 -------------------
        // After the last barrier no wave reads the K/V buffers: output wave w4
        // stages its 32 x D block of O in buffer w4 (bf16, chunk c of row r in
        // slot c ^ (r mod 16)) and stores whole rows, 16 bytes per lane. Stored
        // from the accumulator layout, each instruction would write 8 bytes
        // into each of 32 rows, and lines evicted half-written cost extra
        // write traffic.
        const float lt = l + xor32(l);
        const int qrow = q0 + (lane & 31);
        const bool empty = !(lt > 0.f);
        const float inv = empty ? 0.f : 1.f / lt;
        static_assert(32 * D * 2 == TILE_BYTES, "one output block per K/V buffer");
        MIATTN_LDS uint8_t* stg = (w4 >> 1) ? vbuf(w4 & 1) : kbuf(w4 & 1);
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
              *reinterpret_cast<MIATTN_LDS u32x2*>(sr + 16 * ((4 * dt + r4) ^ (r & 15))) = w;
            }
        }
#pragma unroll
        for (int j = 0; j < 32 * CH / 64; ++j) {
          const int lidx = 64 * j + lane;
          const int r = lidx / CH, ch = lidx % CH;
          const u32x4 w = lds_ld16(stg + r * (2 * D) + 16 * (ch ^ (r & 15)));
          if (q0 + r < L) st16_stream(a.o + ((size_t)(s0 + q0 + r) * Hq + h) * D + 8 * ch, w);
        }
        if (qrow < L && a.lse != nullptr && half == 0)
          a.lse[(size_t)h * a.total_tokens + s0 + qrow] = empty ? kNegInf : (m + log2_hw(lt)) * kLn2;
      }
    }
    // publish the next item; the barrier also closes this item's reads of
    // the K/V buffers (the epilogue staged O there) before the next copies
    if (threadIdx.x == 0) item_slot[(it + 1) & 1] = next;
    __syncthreads();
  }
  // exit count: the last workgroup out zeroes the counters
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(wq + 8, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == gridDim.x - 1) {
    static_assert(kWorkQueueWords == 9, "8 queues and the exit count");
    for (int i = 0; i < kWorkQueueWords; ++i)
      __hip_atomic_exchange(wq + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

}  // namespace miattn
