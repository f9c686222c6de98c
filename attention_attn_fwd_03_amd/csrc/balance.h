// Length-proportional split plan for the paged decode.
//
// With one query token per sequence, a sequence's work is its page count. A
// plan that gives every split of every sequence the same page budget (sized
// from the block-table width) leaves the workgroups of short sequences with
// little work and those of the longest ones with the most, and the launch
// lasts as long as its longest workgroup. Here every group holds C
// consecutive pages of one sequence (its last group may hold fewer):
// sequence b with n_b pages gets s_b = ceil(n_b / C) groups, and C is the
// smallest group size for which the batch needs at most U groups. With T
// pages in all, C lies in [ceil(T / U), ceil(T / (U - B))] (the upper end
// always fits: sum ceil(n_b / C) <= T / C + B), and a binary search over that
// range finds it; with B >= U, C is the longest sequence (one group each).
// Groups are numbered sequence by sequence: group s of sequence b is group
// start_b + s, start_b = s_0 + ... + s_(b-1).
//
// The plan is a function of seq_lens only. One wave derives it with
// wave-wide reductions and scans over the batch, 64 sequences per step; the
// split kernel looks up its group, the combine its sequence, with the same
// operations in the same order, so both see the same plan.
#pragma once
#include "common.h"

namespace miattn {

struct SplitPlan {
  int b;        // sequence (-1: no such group / sequence)
  int s;        // group within the sequence (group lookups)
  int count;    // s_b
  int start;    // index of the sequence's first group
  int n_pages;  // n_b
  int group_pages;  // C
};

__device__ __forceinline__ int plan_pages(const int32_t* seq_lens, int i, int max_pages) {
  int L = seq_lens[i];
  L = L < 0 ? 0 : (L > max_pages * 16 ? max_pages * 16 : L);
  return (L + 15) / 16;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

__device__ __forceinline__ int wave_incl_scan_i32(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) {
    const int o = __shfl_xor(v, m);
    v = v > o ? v : o;
  }
  return v;
}

// Page count of sequence i = base + lane; batches of up to 64 sequences
// (one step) reuse the value loaded once, larger ones reload per step.
struct PlanLanes {
  const int32_t* seq_lens;
  int batch, max_pages, lane, n0;   // n0: page count of sequence lane (first step)
  __device__ int pages(int base) const {
    if (base == 0) return n0;
    const int i = base + lane;
    return i < batch ? plan_pages(seq_lens, i, max_pages) : 0;
  }
};

// groups the batch needs with groups of C pages
__device__ __forceinline__ int plan_groups(const PlanLanes& pl, int C) {
  int total = 0;
  for (int base = 0; base < pl.batch; base += 64) total += wave_sum_i32((pl.pages(base) + C - 1) / C);
  return total;
}

// The group size C of the plan (see above); at least 1.
__device__ inline int plan_group_pages(const PlanLanes& pl, int units) {
  int T = 0, nmax = 0;
  for (int base = 0; base < pl.batch; base += 64) {
    const int n = pl.pages(base);
    T += wave_sum_i32(n);
    const int m = wave_max_i32(n);
    nmax = m > nmax ? m : nmax;
  }
  if (T == 0) return 1;
  if (units <= pl.batch) return nmax;
  int lo = (T + units - 1) / units;                          // sum_b ceil(n_b / C) >= T / C
  int hi = (T + (units - pl.batch) - 1) / (units - pl.batch);  // always fits
  if (hi > nmax) hi = nmax > lo ? nmax : lo;
  while (lo < hi) {
    const int mid = (lo + hi) / 2;
    if (plan_groups(pl, mid) <= units) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// by_group: find group `key` (0 <= key); otherwise sequence `key`. count is
// s_b, start the index of b's first group, n_pages n_b; the group's pages are
// [s C, min((s + 1) C, n_b)) with C = p.group_pages.
__device__ inline SplitPlan balanced_plan(const int32_t* seq_lens, int batch, int max_pages, int units, int key,
                                          bool by_group) {
  const int lane = lane_id();
  const PlanLanes pl = {seq_lens, batch, max_pages, lane, lane < batch ? plan_pages(seq_lens, lane, max_pages) : 0};
  const int C = plan_group_pages(pl, units);
  SplitPlan p = {-1, 0, 0, 0, 0, C};
  int run = 0;
  for (int base = 0; base < batch; base += 64) {
    const int i = base + lane;
    const int n = pl.pages(base);
    const int s = (n + C - 1) / C;
    const int incl = wave_incl_scan_i32(s, lane);
    const int excl = run + incl - s;
    const bool hit = i < batch && (by_group ? (key >= excl && key < excl + s) : (i == key));
    const uint64_t m = __builtin_amdgcn_ballot_w64(hit);
    if (m != 0) {
      const int src = (int)__builtin_ctzll(m);
      p.b = base + src;
      p.count = __builtin_amdgcn_readlane(s, src);
      p.start = __builtin_amdgcn_readlane(excl, src);
      p.n_pages = __builtin_amdgcn_readlane(n, src);
      p.s = by_group ? key - p.start : 0;
      break;
    }
    run += __builtin_amdgcn_readlane(incl, 63);
  }
  return p;
}

// Writes the plan's per-sequence table: start_b at table[b], s_b at
// table[batch + b] (one wave; C from balanced_plan).
__device__ inline void write_plan_table(const int32_t* seq_lens, int batch, int max_pages, int C, int32_t* table) {
  const int lane = lane_id();
  int run = 0;
  for (int base = 0; base < batch; base += 64) {
    const int i = base + lane;
    const int n = i < batch ? plan_pages(seq_lens, i, max_pages) : 0;
    const int s = (n + C - 1) / C;
    const int incl = wave_incl_scan_i32(s, lane);
    if (i < batch) {
      table[i] = run + incl - s;
      table[batch + i] = s;
    }
    run += __builtin_amdgcn_readlane(incl, 63);
  }
}

}  // namespace miattn
