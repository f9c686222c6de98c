// Log-sum-exp merge of split partials ("Why your local LLM feels dumber than
// it is", section "Backend names expand into four decode algorithms",
// FlashAttention 2 entry: fp32 normalised partial outputs weighted by
// exp(LSE_s - max LSE)).
//
// Each workgroup owns one output row and up to 4 * cols of its columns (cols
// float4 columns, chosen by the host so that even a few rows give enough
// workgroups); each thread owns four consecutive columns and a residue class
// of splits. Partial sums are folded through LDS in a fixed order, so the
// result does not depend on scheduling. Empty splits (LSE = -inf) are skipped; an all-empty row gives
// O = 0 and LSE = -inf.
#pragma once
#include "balance.h"
#include "common.h"

namespace miattn {

struct CombineArgs {
  const float* part_o;    // [rows, S, D]
  const float* part_lse;  // [rows, S]
  void* o;                // [rows, D] bf16 or fp32
  float* lse;             // [rows] or null
  int rows;
  int num_splits;
  int head_dim;
  int out_bf16;
  int cols;               // float4 columns per workgroup (4 .. 32, power of two)
  // decode partials in balanced groups (balance.h): row = b * Hq + h reads
  // groups start_b .. start_b + s_b - 1 at [group][Hq][D], start_b and s_b
  // from plan_table ([2][batch], written by the split kernel); null: the
  // [rows][num_splits][D] layout
  const int32_t* plan_table;
  int batch;
  int num_q_heads;
};

// Block-wide max or sum of one float per thread (256 threads): a butterfly
// inside each wave (every lane ends with the same value: each step adds the
// same two numbers in every lane), then the four wave results in wave order.
__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) {
    const float o = __shfl_xor(v, m);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  __syncthreads();   // red may still be read by a previous call
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < 4; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  return r;
}

constexpr int kCombineCols = 32;   // most float4 columns per workgroup (128 output columns)
constexpr int kCombineUnroll = 8;  // independent partial loads in flight per thread

// Float4 columns per combine workgroup: 32 unless that leaves fewer than 512
// workgroups (two per compute unit), then halved down to 4 (64 split groups).
inline int combine_cols(long rows, int head_dim) {
  const int dq = head_dim / 4;
  int cols = kCombineCols;
  while (cols > 4 && rows * ((dq + cols - 1) / cols) < 512) cols >>= 1;
  return cols;
}

// This row's partials: S_row of them, LSE s at pl[s * ls], output s at
// po + s * os (the [rows][S][D] layout, or the balanced groups' layout).
struct RowPartials {
  int S_row;
  const float* pl;
  const float* po;
  size_t ls, os;
};
__device__ __forceinline__ RowPartials row_partials(const CombineArgs& a, int row) {
  RowPartials r;
  const int D = a.head_dim;
  r.S_row = a.num_splits;
  r.pl = a.part_lse + (size_t)row * a.num_splits;
  r.po = a.part_o + (size_t)row * a.num_splits * D;
  r.ls = 1;
  r.os = D;
  if (a.plan_table != nullptr) {
    const int Hq = a.num_q_heads;
    const int b = row / Hq;
    r.S_row = a.plan_table[a.batch + b];
    const size_t first = (size_t)a.plan_table[b] * Hq + row % Hq;
    r.pl = a.part_lse + first;
    r.po = a.part_o + first * D;
    r.ls = Hq;
    r.os = (size_t)Hq * D;
  }
  return r;
}

// One output row merged by the whole workgroup (256 threads, every thread
// must call it): ncol_max float4 columns from col0, ncol column lanes x
// NG = 256 / ncol split groups; group g sums splits g, g + NG, ... in
// increasing order, and the groups are folded pairwise in a fixed order.
__device__ __forceinline__ void combine_row_block(const CombineArgs& a, int row, int col0, int ncol_max,
                                                  float* red, f32x4* part, float* wpart) {
  const int D = a.head_dim;
  const int DQ = D / 4;
  const int ncol = DQ - col0 < ncol_max ? DQ - col0 : ncol_max;
  const int NG = 256 / ncol;
  const int t = threadIdx.x;
  const int c = col0 + t % ncol;
  const int gi = t / ncol;
  const RowPartials rp = row_partials(a, row);
  const int S_row = rp.S_row;
  const float* pl = rp.pl;
  const float* po = rp.po;
  const size_t ls = rp.ls, os = rp.os;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};

  float M, W;
  f32x4 acc = z;
  if (S_row <= NG * kCombineUnroll) {
    // Every thread's splits (gi, gi + NG, ...) fit one batch: their loads are
    // issued before the max is known; the weight sums travel with the
    // partial sums through the fold below.
    f32x4 v[kCombineUnroll];
    float x[kCombineUnroll];
    float mx = kNegInf;
#pragma unroll
    for (int u = 0; u < kCombineUnroll; ++u) {
      const int s = gi + u * NG;
      const bool ok = gi < NG && s < S_row;
      x[u] = ok ? pl[(size_t)s * ls] : kNegInf;
      v[u] = ok ? *reinterpret_cast<const f32x4*>(po + (size_t)s * os + 4 * c) : z;
      mx = fmaxf(mx, x[u]);
    }
    M = block_reduce(mx, red, true);
    float ws = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int u = 0; u < kCombineUnroll; ++u) {
        const bool skip = x[u] == kNegInf;
        const float w = skip ? 0.f : exp2_hw((x[u] - M) * kLog2e);
        ws += w;
        acc += skip ? z : w * v[u];
      }
    }
    part[t] = acc;
    wpart[t] = ws;
    __syncthreads();
    // pairwise fold of the NG groups: in each round group g < n - h adds
    // group g + h (h = ceil(n / 2)); readers and writers never overlap
    for (int n = NG; n > 1;) {
      const int h = (n + 1) >> 1;
      if (gi < n - h) {
        part[t] += part[t + h * ncol];
        wpart[t] += wpart[t + h * ncol];
      }
      n = h;
      __syncthreads();
    }
    W = 0.f;
    if (gi == 0) {
      acc = part[t];
      W = wpart[t];
    }
  } else {
    float mx = kNegInf;
    for (int s = t; s < S_row; s += 256) mx = fmaxf(mx, pl[(size_t)s * ls]);
    M = block_reduce(mx, red, true);
    float ws = 0.f;
    if (M != kNegInf)
      for (int s = t; s < S_row; s += 256) {
        const float x = pl[(size_t)s * ls];
        ws += (x == kNegInf) ? 0.f : exp2_hw((x - M) * kLog2e);
      }
    W = block_reduce(ws, red, false);
    if (M != kNegInf && gi < NG) {
      for (int s0 = gi; s0 < S_row; s0 += NG * kCombineUnroll) {
        f32x4 v[kCombineUnroll];
        float x[kCombineUnroll];
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u) {
          const int s = s0 + u * NG;
          const int sc = s < S_row ? s : S_row - 1;
          x[u] = s < S_row ? pl[(size_t)sc * ls] : kNegInf;
          v[u] = *reinterpret_cast<const f32x4*>(po + (size_t)sc * os + 4 * c);
        }
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u) {
          const float w = exp2_hw((x[u] - M) * kLog2e);
          acc += (x[u] == kNegInf) ? z : w * v[u];
        }
      }
    }
    part[t] = acc;
    __syncthreads();
    for (int n = NG; n > 1;) {   // the pairwise fold above
      const int h = (n + 1) >> 1;
      if (gi < n - h) part[t] += part[t + h * ncol];
      n = h;
      __syncthreads();
    }
    if (gi == 0) acc = part[t];
  }
  if (gi == 0) {
    const bool empty = M == kNegInf || !(W > 0.f);
    const f32x4 sum = empty ? z : acc * (1.f / W);
    if (a.out_bf16) {
      u32x2 w2 = {pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3])};
      *reinterpret_cast<u32x2*>((uint16_t*)a.o + (size_t)row * D + 4 * c) = w2;
    } else {
      *reinterpret_cast<f32x4*>((float*)a.o + (size_t)row * D + 4 * c) = sum;
    }
    if (a.lse != nullptr && c == 0) a.lse[row] = empty ? kNegInf : M + log2_hw(W) * kLn2;
  }
}

// Grid: (rows, ceil(D / (4 cols))): one row and up to cols float4 columns
// per workgroup.
__global__ __launch_bounds__(256) void miattn_combine_kernel(CombineArgs a) {
  __shared__ float red[4];
  __shared__ f32x4 part[256];
  __shared__ float wpart[256];
  combine_row_block(a, blockIdx.x, blockIdx.y * a.cols, a.cols, red, part, wpart);
}

// Most splits per row that one wave merges alone in the row kernel below.
constexpr int kCombineWaveSplits = 16;

// The merge for decode rows with few splits (head_dim 64, 128 or 256): four
// rows per workgroup, one wave per row, no barrier and no LDS. Every lane
// reads all of its row's LSEs, so the max M and the weight sum W (added in
// split order) need no reduction; lane l takes float4 column l mod D/4 of
// the splits s = l / (D/4) + k (64 / (D/4)), and the split groups are folded
// by XOR shuffles (each step adds the same two values in every lane, so all
// lanes agree). A workgroup whose rows have more splits merges them one at a
// time with the whole workgroup, as the kernel above does.
template <int D>
__global__ __launch_bounds__(256) void miattn_combine_rows_kernel(CombineArgs a) {
  __shared__ float red[4];
  __shared__ f32x4 part[256];
  __shared__ float wpart[256];
  constexpr int DQ = D / 4;
  constexpr int NGW = 64 / DQ;                     // split groups per wave
  constexpr int KU = kCombineWaveSplits / NGW;     // partial loads per lane
  static_assert(64 % DQ == 0 && KU >= 1, "head_dim 64, 128 or 256");
  const int r0 = blockIdx.x * 4;
  // the largest split count of the workgroup's rows, read by every wave
  // (a uniform choice without a barrier)
  int smax = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (r0 + i < a.rows) {
      const int sr = row_partials(a, r0 + i).S_row;
      smax = sr > smax ? sr : smax;
    }
  if (smax > kCombineWaveSplits) {
    for (int i = 0; i < 4; ++i)
      if (r0 + i < a.rows) {
        combine_row_block(a, r0 + i, 0, DQ, red, part, wpart);
        __syncthreads();   // this row's fold reads are done before the next row's writes
      }
    return;
  }
  const int row = r0 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int lane = threadIdx.x & 63;
  const int c = lane % DQ, gi = lane / DQ;
  const RowPartials rp = row_partials(a, row);
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  f32x4 v[KU];
  float x[KU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int s = gi + u * NGW;
    const bool ok = s < rp.S_row;
    x[u] = ok ? rp.pl[(size_t)s * rp.ls] : kNegInf;
    v[u] = ok ? *reinterpret_cast<const f32x4*>(rp.po + (size_t)s * rp.os + 4 * c) : z;
  }
  float M = kNegInf;
  for (int s = 0; s < rp.S_row; ++s) M = fmaxf(M, rp.pl[(size_t)s * rp.ls]);
  float W = 0.f;
  f32x4 acc = z;
  if (M != kNegInf) {
    for (int s = 0; s < rp.S_row; ++s) {
      const float xs = rp.pl[(size_t)s * rp.ls];
      W += (xs == kNegInf) ? 0.f : exp2_hw((xs - M) * kLog2e);
    }
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const bool skip = x[u] == kNegInf;
      const float w = skip ? 0.f : exp2_hw((x[u] - M) * kLog2e);
      acc += skip ? z : w * v[u];
    }
  }
#pragma unroll
  for (int m = DQ; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], m);
  if (gi == 0) {
    const bool empty = M == kNegInf || !(W > 0.f);
    const f32x4 sum = empty ? z : acc * (1.f / W);
    if (a.out_bf16) {
      u32x2 w2 = {pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3])};
      *reinterpret_cast<u32x2*>((uint16_t*)a.o + (size_t)row * D + 4 * c) = w2;
    } else {
      *reinterpret_cast<f32x4*>((float*)a.o + (size_t)row * D + 4 * c) = sum;
    }
    if (a.lse != nullptr && c == 0) a.lse[row] = empty ? kNegInf : M + log2_hw(W) * kLn2;
  }
}

}  // namespace miattn

namespace miattn {

// Merges of split statistics records (reference max m_s in log2 units,
// normaliser l_s, and a numerator or normalised partial per column), the
// other three merges of "Why your local LLM feels dumber than it is",
// section "Backend names expand into four decode algorithms":
//   mode 1: numerators and normalisers brought to M = max m_s:
//           O = sum_s num_s 2^(m_s-M) / sum_s l_s 2^(m_s-M);
//   mode 2: normalised partials weighted by their corrected normalisers:
//           O = sum_s o_s l_s 2^(m_s-M) / sum_s l_s 2^(m_s-M);
//   mode 3: an ordered running recurrence over s = 0, 1, ...: the running
//           state (m, l, num) is rescaled to max(m, m_s) and the split added;
//           a running state that is still empty is not rescaled (its weight
//           is 0) and empty splits (m_s = -inf) are skipped.
// LSE = (M + log2 sum) ln 2 in every mode; an all-empty row gives O = 0 and
// LSE = -inf. Modes 1 and 2 reduce in the combine kernel's fixed order; mode 3
// is sequential per column by definition.
struct MergeStatsArgs {
  const float* part_o;   // [rows, S, D]
  const float* part_m;   // [rows, S]
  const float* part_l;   // [rows, S]
  void* o;               // [rows, D] bf16 or fp32
  float* lse;            // [rows] or null
  int rows;
  int num_splits;
  int head_dim;
  int out_bf16;
  int mode;
  int cols;              // float4 columns per workgroup, as for the combine
};

__device__ __forceinline__ void store_row4(const MergeStatsArgs& a, int row, int c, f32x4 v) {
  const int D = a.head_dim;
  if (a.out_bf16) {
    u32x2 w2 = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<u32x2*>((uint16_t*)a.o + (size_t)row * D + 4 * c) = w2;
  } else {
    *reinterpret_cast<f32x4*>((float*)a.o + (size_t)row * D + 4 * c) = v;
  }
}

// Grid: (rows, ceil(D / (4 cols))); 256 threads.
__global__ __launch_bounds__(256) void miattn_merge_stats_kernel(MergeStatsArgs a) {
  __shared__ float red[256];
  __shared__ f32x4 part[256];
  const int row = blockIdx.x;
  const int S = a.num_splits;
  const int D = a.head_dim;
  const int DQ = D / 4;
  const int col0 = blockIdx.y * a.cols;
  const int ncol = DQ - col0 < a.cols ? DQ - col0 : a.cols;
  const int t = threadIdx.x;
  const float* pm = a.part_m + (size_t)row * S;
  const float* pl = a.part_l + (size_t)row * S;
  const float* po = a.part_o + (size_t)row * S * D;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};

  if (a.mode == 3) {
    if (t < ncol) {
      const int c = col0 + t;
      float rm = kNegInf, rl = 0.f;
      f32x4 rn = z;
      // the recurrence is sequential; its loads are not, so they are issued
      // kCombineUnroll splits ahead
      for (int s0 = 0; s0 < S; s0 += kCombineUnroll) {
        float xm[kCombineUnroll], xl[kCombineUnroll];
        f32x4 xv[kCombineUnroll];
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u) {
          const int s = s0 + u < S ? s0 + u : S - 1;
          xm[u] = s0 + u < S ? pm[s] : kNegInf;
          xl[u] = pl[s];
          xv[u] = *reinterpret_cast<const f32x4*>(po + (size_t)s * D + 4 * c);
        }
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u) {
          const float ms = xm[u];
          if (ms == kNegInf) continue;
          const float nm = fmaxf(rm, ms);
          const float keep = (rm == kNegInf) ? 0.f : exp2_hw(rm - nm);
          const float take = exp2_hw(ms - nm);
          rl = rl * keep + xl[u] * take;
          rn = rn * keep + take * xv[u];
          rm = nm;
        }
      }
      const bool empty = !(rl > 0.f);
      store_row4(a, row, c, empty ? z : rn * (1.f / rl));
      if (a.lse != nullptr && c == 0) a.lse[row] = empty ? kNegInf : (rm + log2_hw(rl)) * kLn2;
    }
    return;
  }

  float mx = kNegInf;
  for (int s = t; s < S; s += 256) mx = fmaxf(mx, pm[s]);
  const float M = block_reduce(mx, red, true);
  const bool empty = (M == kNegInf);
  float ws = 0.f;
  if (!empty)
    for (int s = t; s < S; s += 256) ws += (pm[s] == kNegInf) ? 0.f : pl[s] * exp2_hw(pm[s] - M);
  const float W = block_reduce(ws, red, false);

  const int NG = 256 / ncol;
  const int c = col0 + t % ncol;
  const int gi = t / ncol;
  f32x4 acc = z;
  if (!empty && gi < NG) {
    for (int s0 = gi; s0 < S; s0 += NG * kCombineUnroll) {
      float xm[kCombineUnroll], xl[kCombineUnroll];
      f32x4 xv[kCombineUnroll];
#pragma unroll
      for (int u = 0; u < kCombineUnroll; ++u) {
        const int s = s0 + u * NG;
        const int sc = s < S ? s : S - 1;
        xm[u] = s < S ? pm[sc] : kNegInf;
        xl[u] = pl[sc];
        xv[u] = *reinterpret_cast<const f32x4*>(po + (size_t)sc * D + 4 * c);
      }
#pragma unroll
      for (int u = 0; u < kCombineUnroll; ++u) {
        const float f = exp2_hw(xm[u] - M);
        const float w = a.mode == 1 ? f : f * xl[u];
        acc += (xm[u] == kNegInf) ? z : w * xv[u];
      }
    }
  }
  part[t] = acc;
  __syncthreads();
  if (gi == 0) {
    f32x4 sum = part[t];
    for (int k = 1; k < NG; ++k) sum += part[k * ncol + t];
    const bool none = empty || !(W > 0.f);
    store_row4(a, row, c, none ? z : sum * (1.f / W));
    if (a.lse != nullptr && c == 0) a.lse[row] = none ? kNegInf : (M + log2_hw(W)) * kLn2;
  }
}

}  // namespace miattn
