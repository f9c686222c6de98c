// libmiattn host library: argument validation, work planning, workspace and
// kernel launches behind the C ABI declared in include/miattn.h.
#include "../../include/miattn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "backward.h"
#include "combine.h"
#include "decode.h"
#include "prefill.h"
#include "prefill_pp.h"
#include "prefill_pair.h"

// Device scratch of the no-allocation decode entry point: one copy per GPU,
// held until the process ends. In host code `scratch` is only a stand-in for
// the symbol, not a device address: its address on a device comes from
// hipGetSymbolAddress (static_scratch below), once per device, and only that
// address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[MIATTN_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return MIATTN_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
int g_arch_ok[kMaxDevices];          // 0 unknown, 1 gfx950, -1 other

// Library-owned workspaces, one per (device, stream): calls on one stream are
// ordered by that stream, so they may share a buffer; calls on different
// streams never do. A buffer that becomes too small is retired, not freed:
// work already enqueued may still use it, and freeing it safely would need a
// synchronisation. Retired buffers are freed by miattn_release.
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
  unsigned* queue = nullptr;   // work-queue counters of the head_dim-256 prefill
};
std::map<std::pair<int, void*>, Workspace> g_ws;
std::vector<std::pair<int, void*>> g_ws_retired;   // (device, pointer)

bool arch_is_gfx950(int dev) {
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
}

// Current device, checked to be a gfx950; returns the device index or an
// error code.
int current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(MIATTN_ERR_UNSUPPORTED, "no HIP device available");
  }
  if (dev >= kMaxDevices) return fail(MIATTN_ERR_UNSUPPORTED, "device index %d too large", dev);
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_arch_ok[dev] == 0) g_arch_ok[dev] = arch_is_gfx950(dev) ? 1 : -1;
  if (g_arch_ok[dev] < 0) return fail(MIATTN_ERR_UNSUPPORTED, "device %d is not a gfx950", dev);
  return dev;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MIATTN_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return MIATTN_OK;
}

bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }

// --- prefill launches ------------------------------------------------------
template <int D, int QB, int KB, bool CAUSAL, bool PAGED, bool F16V>
void launch_fwd(const miattn::FwdArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((miattn::miattn_prefill_fwd_kernel<D, QB, KB, CAUSAL, PAGED, F16V>), dim3(grid), dim3(256), 0,
                     st, a);
}

template <int D, int QB, int KB, bool PAGED = false, bool F16V = false>
void launch_fwd_c(const miattn::FwdArgs& a, int grid, bool causal, hipStream_t st) {
  if (causal) launch_fwd<D, QB, KB, true, PAGED, F16V>(a, grid, st);
  else launch_fwd<D, QB, KB, false, PAGED, F16V>(a, grid, st);
}

// query blocks of 32 rows per wave in the four-wave kernel: one at every
// head_dim (the template keeps QB as a parameter)
constexpr int fwd_qb(int) { return 1; }

// Dense prefill with head_dim 64 and 128 runs the eight-wave ping-pong kernel
// (two 32-row groups per query tile) when its grid has at least one
// workgroup per compute unit; smaller problems, head_dim 256 and the paged
// (chunked) prefill run the four-wave kernel, which measured faster there
// (half the rows per workgroup: twice the workgroups, half the per-workgroup
// critical path). Both kernels give the same bits.
constexpr bool fwd_pingpong(int d, bool paged) { return d <= 128 && !paged; }

template <int D, int KB, bool F16V>
void launch_fwd_pp(const miattn::FwdArgs& a, int grid, bool causal, hipStream_t st) {
  if (causal)
    hipLaunchKernelGGL((miattn::miattn_prefill_pp_kernel<D, KB, true, F16V>), dim3(grid), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((miattn::miattn_prefill_pp_kernel<D, KB, false, F16V>), dim3(grid), dim3(512), 0, st, a);
}

// Dense bf16 prefill whose P.V product runs on fp16 operands: V is first
// converted to fp16 into a workspace by one streaming pass, and the
// probabilities are rounded to fp16 instead of bf16.
constexpr bool fwd_f16v(int d) { return d >= 256; }

// Query heads of one kv-head group that a prefill workgroup serves together
// (they share every K/V tile it loads): the largest of 4, 2, 1 dividing the
// group size G, so any G runs; the G / NH workgroups of a group read the same
// tiles, the second and later from L2.
int fwd_heads_per_wg(int G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }

// bf16 prefill grid: (head slot, query-tile pair, sequence); `pingpong`:
// the eight-wave kernel's query tiles (twice the four-wave kernel's rows)
long fwd_setup(miattn::FwdArgs& a, int num_seqs, int max_seqlen, int num_q_heads, int num_kv_heads, int head_dim,
               bool pingpong, bool unit_per_tile = false) {
  const int G = num_q_heads / num_kv_heads;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads; a.num_kv_heads = num_kv_heads; a.group = G;
  a.heads_per_wg = fwd_heads_per_wg(G);
  const int QR = 32 * fwd_qb(head_dim) * (4 / a.heads_per_wg) * (pingpong ? 2 : 1);
  const int n_qtiles = (max_seqlen + QR - 1) / QR;
  a.n_pairs = unit_per_tile ? n_qtiles : (n_qtiles + 1) / 2;
  a.n_head_slots = num_kv_heads * (G / a.heads_per_wg);
  return (long)a.n_head_slots * num_seqs * a.n_pairs;
}


template <int D, bool RR = false, bool PF16 = false, bool STUDY = false>
void launch_decode(const miattn::DecodeArgs& a, hipStream_t st) {
  // contiguous splits: splits x head groups x sequences; balanced groups: at
  // most units + batch groups per head group (the surplus exits at once)
  const long groups = a.balance_units > 0 ? (long)a.balance_units + a.batch : (long)a.num_splits * a.batch;
  const unsigned grid = (unsigned)(groups * (a.num_kv_heads / a.heads_per_wg));
  hipLaunchKernelGGL((miattn::miattn_decode_split_kernel<D, RR, PF16, STUDY>), dim3(grid),
                     dim3(miattn::kDecodeThreads), 0, st, a);
}

template <int D>
void launch_decode_study(const miattn::DecodeArgs& a, bool rr, bool pf16, hipStream_t st) {
  if (rr) {
    if (pf16) launch_decode<D, true, true, true>(a, st);
    else launch_decode<D, true, false, true>(a, st);
  } else {
    if (pf16) launch_decode<D, false, true, true>(a, st);
    else launch_decode<D, false, false, true>(a, st);
  }
}

// The library-owned workspace of (dev, stream), grown to at least `need`
// bytes. Growth at least doubles the size, so the retired buffers of a stream
// never add up to more than its current one.
int library_workspace(int dev, hipStream_t stream, size_t need, void** ws, const char* who) {
  std::lock_guard<std::mutex> lk(g_mu);
  Workspace& w = g_ws[std::make_pair(dev, (void*)stream)];
  if (w.bytes < need) {
    size_t bytes = 2 * w.bytes > need ? 2 * w.bytes : need;
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) {
      (void)hipGetLastError();
      return fail(MIATTN_ERR_HIP, "%s: workspace allocation of %zu bytes failed", who, bytes);
    }
    if (w.ptr != nullptr) g_ws_retired.emplace_back(dev, w.ptr);
    w.ptr = p;
    w.bytes = bytes;
  }
  *ws = w.ptr;
  return MIATTN_OK;
}

// The work-queue counters of (dev, stream): allocated and zeroed (by a kernel
// on the stream, so the first launch that uses them is ordered after it) on
// first use; every launch that uses them leaves them zero.
int library_queue(int dev, hipStream_t stream, unsigned** q, const char* who) {
  std::lock_guard<std::mutex> lk(g_mu);
  Workspace& w = g_ws[std::make_pair(dev, (void*)stream)];
  if (w.queue == nullptr) {
    void* p = nullptr;
    if (hipMalloc(&p, miattn::kWorkQueueWords * sizeof(unsigned)) != hipSuccess) {
      (void)hipGetLastError();
      return fail(MIATTN_ERR_HIP, "%s: work-queue allocation failed", who);
    }
    hipLaunchKernelGGL(miattn::miattn_zero_u32_kernel, dim3(1), dim3(64), 0, stream, (unsigned*)p,
                       miattn::kWorkQueueWords);
    if (hipGetLastError() != hipSuccess) {
      (void)hipFree(p);
      return fail(MIATTN_ERR_HIP, "%s: work-queue initialisation failed", who);
    }
    w.queue = (unsigned*)p;
  }
  *q = w.queue;
  return MIATTN_OK;
}

// Device address of `scratch` on each device (null until looked up).
void* g_scratch_ptr[kMaxDevices];

int static_scratch(int dev, void** ptr, const char* who) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return fail(MIATTN_ERR_HIP, "%s: hipGetSymbolAddress of the static scratch failed: %s", who,
                  hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MIATTN_OK;
}

// Checks shared by the decode entry points.
int decode_common_checks(const char* who, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, const int32_t* seq_lens, const void* o,
                         int max_pages_per_seq, int page_size, int num_pages, int num_q_heads, int num_kv_heads,
                         int head_dim, float scale) {
  if (page_size != MIATTN_PAGE_SIZE)
    return fail(MIATTN_ERR_UNSUPPORTED, "%s: page_size must be %d", who, MIATTN_PAGE_SIZE);
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o)
    return fail(MIATTN_ERR_INVALID_ARG, "%s: null pointer", who);
  if (max_pages_per_seq <= 0 || num_pages <= 0)
    return fail(MIATTN_ERR_INVALID_ARG, "%s: max_pages_per_seq and num_pages must be > 0", who);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(MIATTN_ERR_INVALID_ARG, "%s: need Hq > 0, Hkv > 0 and Hq %% Hkv == 0", who);
  if (num_q_heads / num_kv_heads > miattn::kDecodeMaxGroup)
    return fail(MIATTN_ERR_UNSUPPORTED, "%s: Hq/Hkv must be <= %d", who, miattn::kDecodeMaxGroup);
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(MIATTN_ERR_UNSUPPORTED, "%s: head_dim must be 64, 128 or 256", who);
  if (!scale_ok(scale)) return fail(MIATTN_ERR_INVALID_ARG, "%s: scale must be finite and > 0", who);
  return MIATTN_OK;
}

// kv heads per decode workgroup: the largest of 8, 4, 2, 1 dividing Hkv
int decode_heads_per_wg(int hkv) {
  for (int h = 8; h > 1; h >>= 1)
    if (hkv % h == 0) return h;
  return 1;
}

// The split-count rule of "Why your local LLM feels dumber than it is"
// (section "Why FlashAttention 2 selects 54, 62, or 87 groups"). Blocks of
// block_tokens are dealt out in equal runs of ceil(blocks / s), so only the
// distinct run lengths matter; each is represented by the smallest count that
// gives it. Walking the run lengths from the longest down, the count after s
// (run length r) is the first one with a shorter run, ceil(blocks / (r - 1)).
// A count is scored by the filled fraction of its last wave, f = x / ceil(x)
// with x = work_units * s / capacity; the smallest count scoring at least
// threshold times the best score is returned.
int split_rule(long total_tokens, long work_units, long cu_count, long wg_per_cu, long block_tokens,
               long max_splits, double threshold) {
  if (total_tokens <= 0 || work_units <= 0 || cu_count <= 0 || wg_per_cu <= 0 || block_tokens <= 0 ||
      max_splits <= 0)
    return MIATTN_ERR_INVALID_ARG;
  const long blocks = (total_tokens + block_tokens - 1) / block_tokens;
  const long capacity = cu_count * wg_per_cu;
  const long limit = std::min(std::min(max_splits, capacity), blocks);
  auto fill = [&](long s) {
    const long units = work_units * s;
    const long waves = (units + capacity - 1) / capacity;
    return (double)units / (double)(waves * capacity);
  };
  std::vector<std::pair<long, double>> cand;   // (count, score), counts rising
  for (long s = 1; s <= limit;) {
    cand.emplace_back(s, fill(s));
    const long run = (blocks + s - 1) / s;
    if (run <= 1) break;
    s = (blocks + run - 2) / (run - 1);
  }
  double best = 0.0;
  for (const auto& c : cand) best = std::max(best, c.second);
  for (const auto& c : cand)
    if (c.second >= threshold * best) return (int)c.first;
  return 1;
}

// MI355X decode capacity: 256 compute units, one 8-wave split workgroup
// resident per unit, splits counted in 16-token pages, at most 256 splits. The
// decode is HBM-bound and its combine is cheap, so the policy takes the
// smallest split count with the best efficiency (the pages' rule settles for
// 85% of it to save merge work).
constexpr int kCUs = 256;
// Smallest batch x block-table width (in tokens) for which num_splits == 0
// uses the length-proportional plan: measured, the plan's per-workgroup
// start-up costs 1.5-3.7 us, which only launches of this size repay.
constexpr long kDecodePlanMinTokens = 1L << 17;
constexpr int kDecodeWgPerCu = 1;
constexpr int kMaxSplits = 256;
constexpr double kPagesRuleThreshold = 0.85;
constexpr double kDecodePolicyThreshold = 1.0;

}  // namespace

extern "C" {

int miattn_version(void) { return 100; }

const char* miattn_last_error(void) { return g_last_error.c_str(); }

int miattn_device_supported(int device) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  if (device < 0 || device >= n || device >= kMaxDevices) return 0;
  return arch_is_gfx950(device) ? 1 : 0;
}

void miattn_release(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) {
    (void)hipGetLastError();
    return;
  }
  for (auto& kv : g_ws) {
    if (kv.second.ptr != nullptr) g_ws_retired.emplace_back(kv.first.first, kv.second.ptr);
    if (kv.second.queue != nullptr) g_ws_retired.emplace_back(kv.first.first, (void*)kv.second.queue);
  }
  g_ws.clear();
  for (auto& r : g_ws_retired) {
    (void)hipSetDevice(r.first);
    (void)hipFree(r.second);
  }
  g_ws_retired.clear();
  (void)hipSetDevice(cur);
}

int miattn_split_heuristic(int total_tokens, int work_units, int cu_count, int wg_per_cu, int block_tokens,
                           int max_splits) {
  const int r = split_rule(total_tokens, work_units, cu_count, wg_per_cu, block_tokens, max_splits,
                           kPagesRuleThreshold);
  if (r < 0) return fail(r, "split heuristic: all arguments must be positive");
  return r;
}

int miattn_decode_pick_splits(int batch, int num_kv_heads, int max_seq_len) {
  if (batch <= 0 || num_kv_heads <= 0 || max_seq_len <= 0) return 1;
  const long work = (long)batch * (num_kv_heads / decode_heads_per_wg(num_kv_heads));
  return split_rule(max_seq_len, work, kCUs, kDecodeWgPerCu, MIATTN_PAGE_SIZE, kMaxSplits, kDecodePolicyThreshold);
}

size_t miattn_decode_workspace_bytes(int batch, int num_q_heads, int head_dim, int num_splits) {
  if (batch <= 0 || num_q_heads <= 0 || head_dim <= 0 || num_splits == 1 || num_splits < 0) return 0;
  // num_splits == 0: the library policy, at most kCUs + batch groups per head
  const size_t groups = num_splits == 0 ? (size_t)kCUs + batch : (size_t)batch * num_splits;
  const size_t bytes = groups * num_q_heads * ((size_t)head_dim + 1) * sizeof(float) +
                       (num_splits == 0 ? 2 * (size_t)batch * sizeof(int32_t) : 0);
  return (bytes + 255) & ~(size_t)255;
}

int miattn_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens,
                    int num_q_heads, int num_kv_heads, int head_dim, float scale, int causal, int dtype,
                    void* stream) {
  if (num_seqs < 0 || max_seqlen < 0 || total_tokens < 0)
    return fail(MIATTN_ERR_INVALID_ARG, "attn_fwd: negative size");
  if (num_seqs == 0 || total_tokens == 0) return ok();
  if (!q || !k || !v || !o || !cu_seqlens) return fail(MIATTN_ERR_INVALID_ARG, "attn_fwd: null pointer");
  if (max_seqlen <= 0) return fail(MIATTN_ERR_INVALID_ARG, "attn_fwd: max_seqlen must be > 0");
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(MIATTN_ERR_INVALID_ARG, "attn_fwd: need Hq > 0, Hkv > 0 and Hq %% Hkv == 0");
  if (causal != 0 && causal != 1) return fail(MIATTN_ERR_INVALID_ARG, "attn_fwd: causal must be 0 or 1");
  if (!scale_ok(scale)) return fail(MIATTN_ERR_INVALID_ARG, "attn_fwd: scale must be finite and > 0");
  if (dtype != MIATTN_BF16 && dtype != MIATTN_FP32)
    return fail(MIATTN_ERR_UNSUPPORTED, "attn_fwd: unknown dtype %d", dtype);
  const int G = num_q_heads / num_kv_heads;
  if (dtype == MIATTN_BF16) {
    if (head_dim != 64 && head_dim != 128 && head_dim != 256)
      return fail(MIATTN_ERR_UNSUPPORTED, "attn_fwd: bf16 head_dim must be 64, 128 or 256");
  } else if (head_dim != 64) {
    return fail(MIATTN_ERR_UNSUPPORTED, "attn_fwd: fp32 head_dim must be 64");
  }
  const int dev = current_device();
  if (dev < 0) return dev;
  hipStream_t st = (hipStream_t)stream;
  const float c = scale * miattn::kLog2e;

  if (dtype == MIATTN_FP32) {
    miattn::FwdF32Args a;
    a.q = (const float*)q; a.k = (const float*)k; a.v = (const float*)v;
    a.o = (float*)o; a.lse = lse; a.cu_seqlens = cu_seqlens;
    a.num_seqs = num_seqs; a.total_tokens = total_tokens;
    a.num_q_heads = num_q_heads; a.num_kv_heads = num_kv_heads; a.group = G;
    a.n_qtiles = (max_seqlen + 31) / 32; a.c = c;
    const long grid = (long)num_q_heads * num_seqs * a.n_qtiles;
    if (grid > 0x7fffffffL) return fail(MIATTN_ERR_INVALID_ARG, "attn_fwd: problem too large");
    if (causal)
      hipLaunchKernelGGL((miattn::miattn_prefill_fwd_f32_kernel<true>), dim3((unsigned)grid), dim3(512), 0, st, a);
    else
      hipLaunchKernelGGL((miattn::miattn_prefill_fwd_f32_kernel<false>), dim3((unsigned)grid), dim3(512), 0, st, a);
    const int r = check_launch("prefill fp32");
    return r ? r : ok();
  }

  miattn::FwdArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o; a.lse = lse; a.cu_seqlens = cu_seqlens;
  a.total_tokens = total_tokens;
  a.c = c;
  a.seq_lens_k = nullptr; a.block_table = nullptr; a.max_pages = 0; a.num_pages = 0;
  a.queue = nullptr;
  bool pp = fwd_pingpong(head_dim, false);
  // head_dim 256 (pair kernel): one query tile per work item
  long grid = fwd_setup(a, num_seqs, max_seqlen, num_q_heads, num_kv_heads, head_dim, pp, head_dim == 256);
  if (pp && grid < kCUs) {
    pp = false;
    grid = fwd_setup(a, num_seqs, max_seqlen, num_q_heads, num_kv_heads, head_dim, pp);
  }
  if (grid > 0x7fffffffL) return fail(MIATTN_ERR_INVALID_ARG, "attn_fwd: problem too large");
  const bool cz = causal != 0;
  if (fwd_f16v(head_dim)) {
    // V -> fp16 into the stream's library-owned workspace, then the kernel
    // reads that copy
    const long n8 = (long)total_tokens * num_kv_heads * head_dim / 8;
    void* ws = nullptr;
    const int rw = library_workspace(dev, st, (size_t)n8 * 16, &ws, "attn_fwd");
    if (rw) return rw;
    const long blocks = std::min((n8 + 255) / 256, 4096L);
    hipLaunchKernelGGL(miattn::miattn_bf16_to_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const uint16_t*)v, (uint16_t*)ws, n8);
    a.v = (const uint16_t*)ws;
  }
  static_assert(!fwd_f16v(64) && !fwd_f16v(128) && fwd_f16v(256), "P.V precision by head_dim");
  switch (head_dim) {
    case 64:
      if (pp) launch_fwd_pp<64, 2, false>(a, (int)grid, cz, st);
      else launch_fwd_c<64, fwd_qb(64), 2, false, false>(a, (int)grid, cz, st);
      break;
    case 128:
      if (pp) launch_fwd_pp<128, 2, false>(a, (int)grid, cz, st);
      else launch_fwd_c<128, fwd_qb(128), 2, false, false>(a, (int)grid, cz, st);
      break;
    default: {
      // head_dim 256: pairs of specialised waves, one query tile per work
      // item; a persistent grid (one workgroup per compute unit) draws the
      // `grid` items from the stream's work queues
      const int rq = library_queue(dev, st, &a.queue, "attn_fwd");
      if (rq) return rq;
      const unsigned wgs = (unsigned)std::min(grid, (long)kCUs);
      if (cz)
        hipLaunchKernelGGL((miattn::miattn_prefill_pair_kernel<true>), dim3(wgs), dim3(512), 0, st, a);
      else
        hipLaunchKernelGGL((miattn::miattn_prefill_pair_kernel<false>), dim3(wgs), dim3(512), 0, st, a);
      break;
    }
  }
  const int r = check_launch("prefill bf16");
  return r ? r : ok();
}

int miattn_attn_fwd_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                          const int32_t* cu_seqlens_q, const int32_t* seq_lens_k, const int32_t* block_table,
                          int num_seqs, int max_seqlen_q, int total_q, int max_pages_per_seq, int page_size,
                          int num_pages, int num_q_heads, int num_kv_heads, int head_dim, float scale,
                          int causal, void* stream) {
  if (num_seqs < 0 || max_seqlen_q < 0 || total_q < 0)
    return fail(MIATTN_ERR_INVALID_ARG, "attn_fwd_paged: negative size");
  if (page_size != MIATTN_PAGE_SIZE)
    return fail(MIATTN_ERR_UNSUPPORTED, "attn_fwd_paged: page_size must be %d", MIATTN_PAGE_SIZE);
  if (num_seqs == 0 || total_q == 0) return ok();
  if (!q || !k_cache || !v_cache || !o || !cu_seqlens_q || !seq_lens_k || !block_table)
    return fail(MIATTN_ERR_INVALID_ARG, "attn_fwd_paged: null pointer");
  if (max_seqlen_q <= 0) return fail(MIATTN_ERR_INVALID_ARG, "attn_fwd_paged: max_seqlen_q must be > 0");
  if (max_pages_per_seq <= 0 || num_pages <= 0)
    return fail(MIATTN_ERR_INVALID_ARG, "attn_fwd_paged: max_pages_per_seq and num_pages must be > 0");
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(MIATTN_ERR_INVALID_ARG, "attn_fwd_paged: need Hq > 0, Hkv > 0 and Hq %% Hkv == 0");
  if (causal != 0 && causal != 1) return fail(MIATTN_ERR_INVALID_ARG, "attn_fwd_paged: causal must be 0 or 1");
  if (!scale_ok(scale)) return fail(MIATTN_ERR_INVALID_ARG, "attn_fwd_paged: scale must be finite and > 0");
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(MIATTN_ERR_UNSUPPORTED, "attn_fwd_paged: head_dim must be 64, 128 or 256");
  const int G = num_q_heads / num_kv_heads;
  const int dev = current_device();
  if (dev < 0) return dev;
  hipStream_t st = (hipStream_t)stream;
  miattn::FwdArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k_cache; a.v = (const uint16_t*)v_cache;
  a.o = (uint16_t*)o; a.lse = lse; a.cu_seqlens = cu_seqlens_q;
  a.total_tokens = total_q;
  a.c = scale * miattn::kLog2e;
  a.seq_lens_k = seq_lens_k; a.block_table = block_table;
  a.max_pages = max_pages_per_seq; a.num_pages = num_pages;
  a.queue = nullptr;
  const long grid = fwd_setup(a, num_seqs, max_seqlen_q, num_q_heads, num_kv_heads, head_dim, false, true);
  if (grid > 0x7fffffffL) return fail(MIATTN_ERR_INVALID_ARG, "attn_fwd_paged: problem too large");
  const bool cz = causal != 0;
  switch (head_dim) {
    case 64: launch_fwd_c<64, fwd_qb(64), 2, true>(a, (int)grid, cz, st); break;
    case 128: launch_fwd_c<128, fwd_qb(128), 2, true>(a, (int)grid, cz, st); break;
    default: launch_fwd_c<256, fwd_qb(256), 1, true>(a, (int)grid, cz, st); break;
  }
  const int r = check_launch("prefill paged");
  return r ? r : ok();
}

int miattn_attn_combine(const float* partial_o, const float* partial_lse, int rows, int num_splits,
                        int head_dim, void* o, float* lse, int out_dtype, void* stream) {
  if (rows < 0) return fail(MIATTN_ERR_INVALID_ARG, "attn_combine: rows < 0");
  if (num_splits < 1) return fail(MIATTN_ERR_INVALID_ARG, "attn_combine: num_splits must be >= 1");
  if (head_dim < 4 || head_dim > 1024 || head_dim % 4 != 0)
    return fail(MIATTN_ERR_UNSUPPORTED, "attn_combine: head_dim must be a multiple of 4 in [4, 1024]");
  if (out_dtype != MIATTN_BF16 && out_dtype != MIATTN_FP32)
    return fail(MIATTN_ERR_UNSUPPORTED, "attn_combine: unknown out_dtype %d", out_dtype);
  if (rows == 0) return ok();
  if (!partial_o || !partial_lse || !o) return fail(MIATTN_ERR_INVALID_ARG, "attn_combine: null pointer");
  const int dev = current_device();
  if (dev < 0) return dev;
  miattn::CombineArgs a{};
  a.part_o = partial_o; a.part_lse = partial_lse; a.o = o; a.lse = lse;
  a.rows = rows; a.num_splits = num_splits; a.head_dim = head_dim; a.out_bf16 = out_dtype == MIATTN_BF16;
  a.cols = miattn::combine_cols(rows, head_dim);
  const unsigned chunks = (unsigned)((head_dim / 4 + a.cols - 1) / a.cols);
  hipLaunchKernelGGL(miattn::miattn_combine_kernel, dim3(rows, chunks), dim3(256), 0, (hipStream_t)stream, a);
  const int r = check_launch("combine");
  return r ? r : ok();
}

}  // extern "C"

namespace {

// Where the decode's split partials live.
enum class WsMode { kCaller, kStaticScratch };

// The merge of a decode's split partials (head_dim 64, 128 or 256): one wave
// per row for the balanced groups (whose per-row split counts are only known
// on the device; the kernel merges rows with many splits a workgroup at a
// time) and for up to kCombineWaveSplits contiguous splits, the block form
// for more. The numerics entry's LSE record takes the same choice, so it
// gives the fast path's bits.
void launch_decode_merge(miattn::CombineArgs& c, hipStream_t st) {
  if (c.plan_table != nullptr || c.num_splits <= miattn::kCombineWaveSplits) {
    const unsigned g = (unsigned)((c.rows + 3) / 4);
    switch (c.head_dim) {
      case 64: hipLaunchKernelGGL(miattn::miattn_combine_rows_kernel<64>, dim3(g), dim3(256), 0, st, c); break;
      case 128: hipLaunchKernelGGL(miattn::miattn_combine_rows_kernel<128>, dim3(g), dim3(256), 0, st, c); break;
      default: hipLaunchKernelGGL(miattn::miattn_combine_rows_kernel<256>, dim3(g), dim3(256), 0, st, c); break;
    }
  } else {
    c.cols = miattn::combine_cols((long)c.rows, c.head_dim);
    const unsigned chunks = (unsigned)((c.head_dim / 4 + c.cols - 1) / c.cols);
    hipLaunchKernelGGL(miattn::miattn_combine_kernel, dim3((unsigned)c.rows, chunks), dim3(256), 0, st, c);
  }
}

int decode_paged_impl(const char* who, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* seq_lens, int batch, int max_pages_per_seq,
                      int page_size, int num_pages, int num_q_heads, int num_kv_heads, int head_dim, float scale,
                      int num_splits, WsMode mode, void* workspace, size_t workspace_bytes, void* o, float* lse,
                      void* stream) {
  if (batch < 0) return fail(MIATTN_ERR_INVALID_ARG, "%s: batch < 0", who);
  if (num_splits < 0) return fail(MIATTN_ERR_INVALID_ARG, "%s: num_splits < 0", who);
  if (page_size != MIATTN_PAGE_SIZE)
    return fail(MIATTN_ERR_UNSUPPORTED, "%s: page_size must be %d", who, MIATTN_PAGE_SIZE);
  if (batch == 0) return ok();
  {
    const int r = decode_common_checks(who, q, k_cache, v_cache, block_table, seq_lens, o,
                                       max_pages_per_seq, page_size, num_pages, num_q_heads, num_kv_heads,
                                       head_dim, scale);
    if (r) return r;
  }
  int S = num_splits;
  // num_splits == 0: where the split-count policy would split at all and the
  // launch is large (batch x table width >= kDecodePlanMinTokens), the library
  // splits each sequence into groups proportional to its length (units groups
  // per kv-head group in all); otherwise the policy's contiguous splits
  int units = 0;
  const int n_hg = num_kv_heads / decode_heads_per_wg(num_kv_heads);
  if (S == 0) {
    S = miattn_decode_pick_splits(batch, num_kv_heads, max_pages_per_seq * MIATTN_PAGE_SIZE);
    // (a single sequence's groups are the contiguous splits already; small
    // launches would pay the plan's start-up, ~2 us, for little balance)
    if (S > 1 && batch > 1 && (long)batch * max_pages_per_seq * MIATTN_PAGE_SIZE >= kDecodePlanMinTokens)
      units = kCUs / n_hg > 1 ? kCUs / n_hg : 1;
    // contiguous groups keep within the workspace bound published for
    // num_splits == 0 (kCUs + batch groups per head): batch * S <= kCUs + batch
    else if (S > 1 + kCUs / batch)
      S = 1 + kCUs / batch;
  }
  if (S > max_pages_per_seq) S = max_pages_per_seq;   // more splits than pages would only add empty groups
  if (S < 1) S = 1;
  if ((long)S * num_kv_heads * batch > 0x7fffffffL || (long)(units + batch) * num_kv_heads > 0x7fffffffL)
    return fail(MIATTN_ERR_INVALID_ARG, "%s: splits * Hkv * batch too large", who);
  // balanced groups: partials of units + batch groups, then the plan table
  const size_t need = units > 0 ? ((((size_t)units + batch) * num_q_heads * ((size_t)head_dim + 1) * sizeof(float) +
                                    2 * (size_t)batch * sizeof(int32_t) + 255) & ~(size_t)255)
                                : miattn_decode_workspace_bytes(batch, num_q_heads, head_dim, S);
  if (mode == WsMode::kCaller && workspace != nullptr && workspace_bytes < need)
    return fail(MIATTN_ERR_WORKSPACE, "%s: workspace of %zu bytes, need %zu", who, workspace_bytes, need);
  if (mode == WsMode::kStaticScratch && need > (size_t)MIATTN_NOALLOC_SCRATCH_BYTES)
    return fail(MIATTN_ERR_WORKSPACE, "%s: the split partials need %zu bytes, the static scratch holds %zu", who,
                need, (size_t)MIATTN_NOALLOC_SCRATCH_BYTES);
  const int dev = current_device();
  if (dev < 0) return dev;
  hipStream_t st = (hipStream_t)stream;
  void* ws = workspace;
  if (mode == WsMode::kStaticScratch) {
    ws = nullptr;
    if (need > 0) {
      const int r = static_scratch(dev, &ws, who);
      if (r) return r;
    }
  } else if (need > 0 && ws == nullptr) {
    const int r = library_workspace(dev, st, need, &ws, who);
    if (r) return r;
  }
  miattn::DecodeArgs a{};
  a.q = (const uint16_t*)q; a.k_cache = (const uint16_t*)k_cache; a.v_cache = (const uint16_t*)v_cache;
  a.block_table = block_table; a.seq_lens = seq_lens; a.batch = batch;
  const size_t rows = (size_t)batch * num_q_heads;
  // partials: [rows][S] (contiguous splits) or [units + batch][Hq] (groups)
  const size_t slots = units > 0 ? ((size_t)units + batch) * num_q_heads : rows * (size_t)S;
  a.part_o = S > 1 ? (float*)ws : nullptr;
  a.part_lse = S > 1 ? (float*)ws + slots * head_dim : nullptr;
  a.balance_units = units;
  a.plan_table = units > 0 ? (int32_t*)(a.part_lse + slots) : nullptr;
  a.o = (uint16_t*)o; a.lse = lse;
  a.max_pages = max_pages_per_seq; a.num_pages = num_pages;
  a.num_q_heads = num_q_heads; a.num_kv_heads = num_kv_heads; a.group = num_q_heads / num_kv_heads;
  a.heads_per_wg = decode_heads_per_wg(num_kv_heads);
  a.num_splits = S; a.c = scale * miattn::kLog2e;
  switch (head_dim) {
    case 64: launch_decode<64>(a, st); break;
    case 128: launch_decode<128>(a, st); break;
    default: launch_decode<256>(a, st); break;
  }
  int r = check_launch("decode split");
  if (r) return r;
  if (S > 1) {
    miattn::CombineArgs c{};
    c.part_o = a.part_o; c.part_lse = a.part_lse; c.o = o; c.lse = lse;
    c.rows = (int)rows; c.num_splits = S; c.head_dim = head_dim; c.out_bf16 = 1;
    if (units > 0) {
      c.plan_table = a.plan_table; c.batch = batch; c.num_q_heads = num_q_heads;
    }
    launch_decode_merge(c, st);
    r = check_launch("combine");
    if (r) return r;
  }
  return ok();
}

}  // namespace

extern "C" {

int miattn_attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens, int batch,
                             int max_pages_per_seq, int page_size, int num_pages, int num_q_heads,
                             int num_kv_heads, int head_dim, float scale, int num_splits, void* workspace,
                             size_t workspace_bytes, void* o, float* lse, void* stream) {
  return decode_paged_impl("attn_decode_paged", q, k_cache, v_cache, block_table, seq_lens, batch,
                           max_pages_per_seq, page_size, num_pages, num_q_heads, num_kv_heads, head_dim, scale,
                           num_splits, WsMode::kCaller, workspace, workspace_bytes, o, lse, stream);
}

int miattn_attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_table, const int32_t* seq_lens, int batch,
                                     int max_pages_per_seq, int page_size, int num_pages, int num_q_heads,
                                     int num_kv_heads, int head_dim, float scale, int num_splits, void* o,
                                     float* lse, void* stream) {
  return decode_paged_impl("attn_decode_paged_noalloc", q, k_cache, v_cache, block_table, seq_lens, batch,
                           max_pages_per_seq, page_size, num_pages, num_q_heads, num_kv_heads, head_dim, scale,
                           num_splits, WsMode::kStaticScratch, nullptr, 0, o, lse, stream);
}

namespace {
// row length of the backward's stats arrays: T plus a 32-row tile of slack,
// rounded up to 64
long bwd_t_pad(int total_tokens) { return ((long)total_tokens + 32 + 63) / 64 * 64; }
}  // namespace

size_t miattn_attn_bwd_workspace_bytes(int total_tokens, int num_q_heads, int num_kv_heads, int head_dim) {
  if (total_tokens <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0) return 0;
  const size_t stats = 2 * (size_t)num_q_heads * bwd_t_pad(total_tokens) * sizeof(float);
  const size_t copies = 2 * (size_t)total_tokens * (num_q_heads + num_kv_heads) * head_dim * 2;
  return ((stats + 255) & ~(size_t)255) + ((copies + 255) & ~(size_t)255);
}

int miattn_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens, int num_q_heads,
                    int num_kv_heads, int head_dim, float scale, int causal, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "attn_bwd";
  if (num_seqs < 0 || max_seqlen < 0 || total_tokens < 0) return fail(MIATTN_ERR_INVALID_ARG, "%s: negative size", who);
  if (num_seqs == 0 || total_tokens == 0) return ok();
  if (!q || !k || !v || !o || !dout || !lse || !cu_seqlens || !dq || !dk || !dv)
    return fail(MIATTN_ERR_INVALID_ARG, "%s: null pointer", who);
  if (max_seqlen <= 0) return fail(MIATTN_ERR_INVALID_ARG, "%s: max_seqlen must be > 0", who);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(MIATTN_ERR_INVALID_ARG, "%s: need Hq > 0, Hkv > 0 and Hq %% Hkv == 0", who);
  if (causal != 0 && causal != 1) return fail(MIATTN_ERR_INVALID_ARG, "%s: causal must be 0 or 1", who);
  if (!scale_ok(scale)) return fail(MIATTN_ERR_INVALID_ARG, "%s: scale must be finite and > 0", who);
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(MIATTN_ERR_UNSUPPORTED, "%s: head_dim must be 64, 128 or 256", who);
  const int G = num_q_heads / num_kv_heads;
  if ((long)total_tokens * num_q_heads * head_dim > 0x7fffffffL ||
      2L * num_q_heads * bwd_t_pad(total_tokens) > 0x3fffffffL)
    return fail(MIATTN_ERR_INVALID_ARG, "%s: tensors above 2^31 elements are not supported", who);
  const size_t need = miattn_attn_bwd_workspace_bytes(total_tokens, num_q_heads, num_kv_heads, head_dim);
  if (workspace != nullptr && workspace_bytes < need)
    return fail(MIATTN_ERR_WORKSPACE, "%s: workspace of %zu bytes, need %zu", who, workspace_bytes, need);
  const int dev = current_device();
  if (dev < 0) return dev;
  hipStream_t st = (hipStream_t)stream;
  void* ws = workspace;
  if (ws == nullptr) {
    const int r = library_workspace(dev, st, need, &ws, who);
    if (r) return r;
  }
  const long t_pad = bwd_t_pad(total_tokens);
  const size_t stats_bytes = (2 * (size_t)num_q_heads * t_pad * sizeof(float) + 255) & ~(size_t)255;
  const size_t nq = (size_t)total_tokens * num_q_heads * head_dim;
  const size_t nk = (size_t)total_tokens * num_kv_heads * head_dim;
  miattn::BwdArgs a{};
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.o = (const uint16_t*)o; a.dout = (const uint16_t*)dout; a.lse = lse;
  a.stats = (float*)ws;
  a.q16 = (uint16_t*)((char*)ws + stats_bytes);
  a.do16 = a.q16 + nq;
  a.k16 = a.do16 + nq;
  a.v16 = a.k16 + nk;
  a.dq = (uint16_t*)dq; a.dk = (uint16_t*)dk; a.dv = (uint16_t*)dv;
  a.cu_seqlens = cu_seqlens; a.num_seqs = num_seqs; a.total_tokens = total_tokens; a.t_pad = (int)t_pad;
  a.num_q_heads = num_q_heads; a.num_kv_heads = num_kv_heads; a.group = G;
  a.heads_per_wg = fwd_heads_per_wg(G);
  a.n_head_slots = num_kv_heads * (G / a.heads_per_wg);
  a.c = scale * miattn::kLog2e;
  a.scale = scale;
  const long rows = (long)total_tokens * (num_q_heads + num_kv_heads);
  const int rpb = 256 / (head_dim / 8);
  const unsigned g_prep = (unsigned)((rows + rpb - 1) / rpb);
  // 64-key blocks: two waves of 32 keys per SIMD (head_dim 64, 128), four
  // waves of 16 keys (head_dim 256)
  a.n_kblocks = (max_seqlen + 63) / 64;
  const unsigned g_dkdv = (unsigned)((long)num_kv_heads * a.n_kblocks * num_seqs);
  const int QR = 32 * (4 / a.heads_per_wg);
  a.n_qunits = (max_seqlen + QR - 1) / QR;
  const unsigned g_dq = (unsigned)((long)a.n_head_slots * a.n_qunits * num_seqs);
  const dim3 blk(256);
  if (head_dim == 64) {
    hipLaunchKernelGGL(miattn::miattn_bwd_prep_kernel<64>, dim3(g_prep), blk, 0, st, a);
    if (causal) {
      hipLaunchKernelGGL((miattn::miattn_bwd_dkdv_pair_kernel<64, true>), dim3(g_dkdv), dim3(512), 0, st, a);
      hipLaunchKernelGGL((miattn::miattn_bwd_dq_kernel<64, 2, true>), dim3(g_dq), blk, 0, st, a);
    } else {
      hipLaunchKernelGGL((miattn::miattn_bwd_dkdv_pair_kernel<64, false>), dim3(g_dkdv), dim3(512), 0, st, a);
      hipLaunchKernelGGL((miattn::miattn_bwd_dq_kernel<64, 2, false>), dim3(g_dq), blk, 0, st, a);
    }
  } else if (head_dim == 128) {
    hipLaunchKernelGGL(miattn::miattn_bwd_prep_kernel<128>, dim3(g_prep), blk, 0, st, a);
    if (causal) {
      hipLaunchKernelGGL((miattn::miattn_bwd_dkdv_pair_kernel<128, true>), dim3(g_dkdv), dim3(512), 0, st, a);
      hipLaunchKernelGGL((miattn::miattn_bwd_dq_kernel<128, 2, true>), dim3(g_dq), blk, 0, st, a);
    } else {
      hipLaunchKernelGGL((miattn::miattn_bwd_dkdv_pair_kernel<128, false>), dim3(g_dkdv), dim3(512), 0, st, a);
      hipLaunchKernelGGL((miattn::miattn_bwd_dq_kernel<128, 2, false>), dim3(g_dq), blk, 0, st, a);
    }
  } else {
    hipLaunchKernelGGL(miattn::miattn_bwd_prep_kernel<256>, dim3(g_prep), blk, 0, st, a);
    if (causal) {
      hipLaunchKernelGGL((miattn::miattn_bwd_dkdv_d256_kernel<true>), dim3(g_dkdv), blk, 0, st, a);
      hipLaunchKernelGGL((miattn::miattn_bwd_dq_kernel<256, 1, true>), dim3(g_dq), blk, 0, st, a);
    } else {
      hipLaunchKernelGGL((miattn::miattn_bwd_dkdv_d256_kernel<false>), dim3(g_dkdv), blk, 0, st, a);
      hipLaunchKernelGGL((miattn::miattn_bwd_dq_kernel<256, 1, false>), dim3(g_dq), blk, 0, st, a);
    }
  }
  const int r = check_launch(who);
  return r ? r : ok();
}

size_t miattn_decode_numerics_workspace_bytes(int batch, int num_q_heads, int head_dim, int num_splits) {
  if (batch <= 0 || num_q_heads <= 0 || head_dim <= 0 || num_splits <= 0) return 0;
  const size_t rows = (size_t)batch * num_q_heads;
  const size_t bytes = rows * (size_t)num_splits * ((size_t)head_dim + 2) * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

int miattn_attn_decode_paged_numerics(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* seq_lens, int batch,
                                      int max_pages_per_seq, int page_size, int num_pages, int num_q_heads,
                                      int num_kv_heads, int head_dim, float scale, int num_splits, int numerics,
                                      int tile_pages, void* workspace, size_t workspace_bytes, void* o,
                                      int out_dtype, float* lse, void* stream) {
  const char* who = "attn_decode_paged_numerics";
  if (batch < 0) return fail(MIATTN_ERR_INVALID_ARG, "%s: batch < 0", who);
  if (num_splits < 0) return fail(MIATTN_ERR_INVALID_ARG, "%s: num_splits < 0", who);
  if (numerics & ~0xF) return fail(MIATTN_ERR_UNSUPPORTED, "%s: unknown numerics bits 0x%x", who, numerics);
  if (tile_pages < 0 || tile_pages > 1024 || (tile_pages & (tile_pages - 1)) != 0)
    return fail(MIATTN_ERR_UNSUPPORTED, "%s: tile_pages must be 0 or a power of two <= 1024", who);
  if (out_dtype != MIATTN_BF16 && out_dtype != MIATTN_FP32)
    return fail(MIATTN_ERR_UNSUPPORTED, "%s: unknown out_dtype %d", who, out_dtype);
  if (page_size != MIATTN_PAGE_SIZE)
    return fail(MIATTN_ERR_UNSUPPORTED, "%s: page_size must be %d", who, MIATTN_PAGE_SIZE);
  if (batch == 0) return ok();
  {
    const int r = decode_common_checks(who, q, k_cache, v_cache, block_table, seq_lens, o, max_pages_per_seq,
                                       page_size, num_pages, num_q_heads, num_kv_heads, head_dim, scale);
    if (r) return r;
  }
  const int record = numerics & 3;
  const bool rr = tile_pages > 0;
  int S = num_splits;
  if (S == 0) S = miattn_decode_pick_splits(batch, num_kv_heads, max_pages_per_seq * MIATTN_PAGE_SIZE);
  // more splits than pages (or tiles) would only add empty groups
  const int units = rr ? (max_pages_per_seq + tile_pages - 1) / tile_pages : max_pages_per_seq;
  if (S > units) S = units;
  if (S < 1) S = 1;
  if ((long)S * num_kv_heads * batch > 0x7fffffffL)
    return fail(MIATTN_ERR_INVALID_ARG, "%s: splits * Hkv * batch too large", who);
  const size_t need = miattn_decode_numerics_workspace_bytes(batch, num_q_heads, head_dim, S);
  if (workspace != nullptr && workspace_bytes < need)
    return fail(MIATTN_ERR_WORKSPACE, "%s: workspace of %zu bytes, need %zu", who, workspace_bytes, need);
  const int dev = current_device();
  if (dev < 0) return dev;
  hipStream_t st = (hipStream_t)stream;
  void* ws = workspace;
  if (ws == nullptr) {
    const int r = library_workspace(dev, st, need, &ws, who);
    if (r) return r;
  }
  const size_t rows = (size_t)batch * num_q_heads;
  miattn::DecodeArgs a{};
  a.q = (const uint16_t*)q; a.k_cache = (const uint16_t*)k_cache; a.v_cache = (const uint16_t*)v_cache;
  a.block_table = block_table; a.seq_lens = seq_lens; a.batch = batch;
  a.part_o = (float*)ws;
  a.part_m = a.part_o + rows * (size_t)S * head_dim;
  a.part_l = a.part_m + rows * (size_t)S;
  a.part_lse = a.part_m;
  a.o = nullptr; a.lse = nullptr;
  a.max_pages = max_pages_per_seq; a.num_pages = num_pages;
  a.num_q_heads = num_q_heads; a.num_kv_heads = num_kv_heads; a.group = num_q_heads / num_kv_heads;
  a.heads_per_wg = decode_heads_per_wg(num_kv_heads);
  a.num_splits = S; a.c = scale * miattn::kLog2e;
  a.record = record;
  a.rounded_l = (numerics & MIATTN_NUMERICS_ROUNDED_NORMALIZER) ? 1 : 0;
  a.tile_shift = rr ? __builtin_ctz((unsigned)tile_pages) : 0;
  const bool pf16 = (numerics & MIATTN_NUMERICS_P_FP16) != 0;
  switch (head_dim) {
    case 64: launch_decode_study<64>(a, rr, pf16, st); break;
    case 128: launch_decode_study<128>(a, rr, pf16, st); break;
    default: launch_decode_study<256>(a, rr, pf16, st); break;
  }
  int r = check_launch("decode split (numerics)");
  if (r) return r;
  const int cols = miattn::combine_cols((long)rows, head_dim);
  const unsigned chunks = (unsigned)((head_dim / 4 + cols - 1) / cols);
  if (record == 0) {
    miattn::CombineArgs c{};
    c.part_o = a.part_o; c.part_lse = a.part_lse; c.o = o; c.lse = lse;
    c.rows = (int)rows; c.num_splits = S; c.head_dim = head_dim; c.out_bf16 = out_dtype == MIATTN_BF16;
    launch_decode_merge(c, st);
  } else {
    miattn::MergeStatsArgs m{};
    m.part_o = a.part_o; m.part_m = a.part_m; m.part_l = a.part_l; m.o = o; m.lse = lse;
    m.rows = (int)rows; m.num_splits = S; m.head_dim = head_dim; m.out_bf16 = out_dtype == MIATTN_BF16;
    m.mode = record;
    m.cols = cols;
    hipLaunchKernelGGL(miattn::miattn_merge_stats_kernel, dim3((unsigned)rows, chunks), dim3(256), 0, st, m);
  }
  r = check_launch("merge (numerics)");
  return r ? r : ok();
}

}  // extern "C"
