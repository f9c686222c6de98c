/*
 * libmiattn -- tiled scaled-dot-product attention with an online softmax for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the one defined in "Why your local LLM feels dumber than it
 * is" (section "What attention is trying to calculate"): for a query row i of
 * head h and the keys J(i) it may see,
 *     s_ij = scale * dot(q_i, k_j),   O_i = sum_j exp(s_ij) v_j / sum_j exp(s_ij),
 *     LSE_i = ln sum_j exp(s_ij)      (natural log, in units of the scaled score).
 * It is evaluated tile by tile without materialising the scores, with the
 * running max / running sum rescaling of "Streaming process" (steps 3-8 and its
 * code snippet); the result equals the definition up to rounding order.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     keeps none of them after the call returns. Layouts are row-major with the
 *     last dimension contiguous.
 *   - Query head h reads key/value head g = h / (Hq / Hkv) (contiguous groups).
 *   - `stream` is a hipStream_t (NULL = the default stream). A return value of
 *     MIATTN_OK means the work was enqueued; results are valid once the stream
 *     has been synchronised. The library performs no device synchronisation
 *     and no device-to-host reads.
 *   - All arguments are validated on the host before any HIP call; an invalid
 *     call returns an error code, enqueues nothing and leaves no sticky HIP
 *     error. miattn_last_error() describes the most recent failure of the
 *     calling thread.
 *   - For a fixed problem (shapes, page size and split count) the outputs are
 *     bitwise identical from run to run: no floating-point atomics are used and
 *     every reduction has a fixed order.
 *   - Inputs are not checked for NaN/Inf; non-finite inputs propagate.
 *
 * Library-owned workspaces (workspace == NULL in the calls that take one,
 * and the fp16 copy of V made by miattn_attn_fwd at head_dim 256)
 *   The library keeps one scratch buffer per (device, stream) pair: calls on
 *   the same stream run in stream order and share it; calls on different
 *   streams use different buffers, so they may overlap. A buffer that is too
 *   small for a call is replaced by a larger one (at least twice the size);
 *   the old one is kept, not freed, because work already enqueued may still
 *   read it, so growth needs no synchronisation. All of them are freed by
 *   miattn_release. The buffer of a stream handle is reused by a later stream
 *   that gets the same handle value: destroy a stream only once the library
 *   calls enqueued on it have finished.
 *   miattn_attn_fwd at head_dim 256 also keeps, per (device, stream), nine
 *   32-bit work-queue counters (allocated and zeroed on the stream by the
 *   first such call; each launch leaves them zero again), under the same
 *   rules: no synchronisation, freed by miattn_release.
 *   HIP graph capture: the calls enqueue kernels only (no memset, copy or
 *   synchronisation), so they can be captured once the capturing stream's
 *   library-owned buffers exist: make each call once, eagerly, on that
 *   stream before capturing, so that no call allocates device memory while
 *   the stream is capturing. Replays and eager calls on the stream share the
 *   buffers in stream order.
 */
#ifndef MIATTN_H
#define MIATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define MIATTN_OK                 0
#define MIATTN_ERR_INVALID_ARG   (-1)  /* bad pointer, size or flag              */
#define MIATTN_ERR_UNSUPPORTED   (-2)  /* dtype / head_dim / device not handled  */
#define MIATTN_ERR_HIP           (-3)  /* a HIP call or kernel launch failed     */
#define MIATTN_ERR_WORKSPACE     (-4)  /* caller workspace smaller than needed   */

/* element types */
#define MIATTN_BF16 0
#define MIATTN_FP32 1

#define MIATTN_PAGE_SIZE 16            /* tokens per KV-cache page               */

/*
 * miattn_attn_fwd -- prefill / dense forward over packed variable-length
 * sequences (FlashAttention forward: "Streaming process" steps 3-8 and code
 * snippet; the causal GQA cells of "GPU Datapath: Where Every Byte Moves",
 * section C; varlen packing through cu_seqlens as in that page's section
 * "Measuring the Real Kernels, One at a Time").
 *
 *   q    [total_tokens, Hq,  D]  dtype
 *   k, v [total_tokens, Hkv, D]  dtype
 *   o    [total_tokens, Hq,  D]  dtype        (written)
 *   lse  [Hq, total_tokens]      float32      (written; may be NULL)
 *   cu_seqlens [num_seqs + 1]    int32, device; sequence b occupies token rows
 *        [cu_seqlens[b], cu_seqlens[b+1]). Must be non-decreasing, start at 0
 *        and end at total_tokens, and no sequence may exceed max_seqlen. Rows
 *        outside these promises are clamped so that no access leaves the
 *        buffers, but their results are unspecified.
 *   num_seqs, max_seqlen, total_tokens: host integers that size the grid.
 *   scale: finite and > 0 (scores are scale * q.k).
 *   causal: 0 = every key of the sequence; 1 = key j <= query i (positions
 *        counted from each sequence's start; queries and keys coincide).
 *   dtype: MIATTN_BF16 with head_dim 64, 128 or 256, or MIATTN_FP32 with
 *        head_dim 64; any Hq/Hkv. bf16 inputs are multiplied on bf16 MFMA with fp32
 *        accumulation; softmax state is fp32; O is rounded to bf16 once at
 *        the end; the row sums add the unrounded fp32 probabilities. In the
 *        P.V product the probabilities enter rounded to bf16 at head_dim 64
 *        and 128; at head_dim 256 they enter rounded to fp16 and V is first
 *        converted to fp16 by one streaming pass into the library-owned
 *        workspace of the stream (exact for |v| <= 65504, the domain of V at
 *        head_dim 256; values below 2^-14 become fp16 subnormals, error at
 *        most 2^-25). fp32 inputs stay fp32 throughout (fp32 MFMA).
 *   LSE_i = max_j s_ij + ln sum_j exp(s_ij - max_j s_ij).
 * num_seqs == 0 or total_tokens == 0 is a no-op returning MIATTN_OK.
 */
int miattn_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens,
                    int num_q_heads, int num_kv_heads, int head_dim, float scale, int causal,
                    int dtype, void* stream);

/*
 * miattn_attn_fwd_paged -- chunked prefill: each sequence's new query chunk
 * attends to that sequence's keys/values held in a paged KV cache, the same
 * cache layout and block table the decode path reads ("GPU Datapath", section
 * D: 16-token pages in any order, reached through a block table; the varlen
 * entry with a block table of section "Measuring the Real Kernels, One at a
 * Time"). The chunk is the last Lq tokens of the sequence, whose Lk cached
 * tokens already include the chunk's own keys.
 *
 *   q, o     [total_q, Hq, D] bf16 (o written); packed by cu_seqlens_q
 *   lse      [Hq, total_q] float32 (written; may be NULL)
 *   k_cache, v_cache [num_pages, 16, Hkv, D] bf16
 *   cu_seqlens_q [num_seqs + 1] int32, device: sequence b's queries are rows
 *            [cu_seqlens_q[b], cu_seqlens_q[b+1]), Lq of them
 *   seq_lens_k [num_seqs] int32, device: Lk, the cached tokens of sequence b
 *            (normally Lk >= Lq); logical page p of sequence b is physical
 *            page block_table[b * max_pages_per_seq + p]
 *   causal: 0 = every query sees all Lk keys; 1 = query i (0-based within the
 *            chunk) sees keys j <= i + Lk - Lq (queries aligned to the end of
 *            the sequence). A query that sees no key gets O = 0, LSE = -inf.
 *   page_size must be MIATTN_PAGE_SIZE; head_dim 64, 128 or 256; any Hq/Hkv.
 *   Numerics as miattn_attn_fwd with bf16.
 *   num_seqs, max_seqlen_q, total_q, max_pages_per_seq, num_pages: host
 *   integers that size the grid and bound the indices.
 * Robustness: Lk is clamped to [0, max_pages_per_seq * 16]; block-table
 * entries outside [0, num_pages) read page 0. Such inputs never fault, but
 * their results are unspecified. With Lq == Lk, an in-order table and a
 * contiguous cache this is exactly miattn_attn_fwd.
 */
int miattn_attn_fwd_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                          const int32_t* cu_seqlens_q, const int32_t* seq_lens_k, const int32_t* block_table,
                          int num_seqs, int max_seqlen_q, int total_q, int max_pages_per_seq, int page_size,
                          int num_pages, int num_q_heads, int num_kv_heads, int head_dim, float scale,
                          int causal, void* stream);

/*
 * miattn_attn_decode_paged -- one query token per sequence against a paged
 * KV cache ("GPU Datapath", section D: block table of 16-token pages, pages in
 * any order), evaluated split-KV: split s of every sequence covers logical
 * pages [s * P, (s + 1) * P) with P = ceil(max_pages_per_seq / num_splits)
 * (equal-size, page-aligned groups sized from the block-table width; the
 * pages past a sequence's own length are skipped, so its last groups may be
 * short or empty), each group yields a normalised partial output and its
 * log-sum-exp, and the groups are merged by log-sum-exp weights ("Why your
 * local LLM feels dumber than it is", sections "Why the calculation is split
 * into groups" and "Backend names expand into four decode algorithms",
 * FlashAttention 2 entry). An empty group contributes weight 0.
 *
 *   q        [batch, Hq, D]                         bf16
 *   k_cache, v_cache [num_pages, 16, Hkv, D]        bf16
 *   block_table [batch, max_pages_per_seq]          int32, device: logical page
 *            p of sequence b is physical page block_table[b, p]
 *   seq_lens [batch]                                int32, device: tokens
 *            cached for each sequence (the query sees all of them)
 *   o        [batch, Hq, D] bf16 (written); lse [batch, Hq] float32 (written;
 *            may be NULL). A sequence of length 0 gives o = 0, lse = -inf.
 *   page_size must be MIATTN_PAGE_SIZE; head_dim 64, 128 or 256; Hq/Hkv <= 16
 *            (MIATTN_ERR_UNSUPPORTED otherwise).
 *   num_splits: >= 1 to fix the split count (the contiguous groups above;
 *            counts above max_pages_per_seq are lowered to it), or 0 for the
 *            library's plan: where miattn_decode_pick_splits would split at all,
 *            the batch holds more than one sequence and batch *
 *            max_pages_per_seq * page_size >= 2^17, every group holds the
 *            same number C of consecutive pages of one sequence (its last group
 *            fewer), C being the smallest size for which the batch needs at
 *            most 256 / (kv-head groups of a workgroup) groups, so sequences of
 *            any length mix share the work evenly (the plan depends on
 *            seq_lens only); otherwise the pick_splits count of contiguous
 *            groups, at most 1 + 256 / batch. Bitwise reproducibility holds for a fixed num_splits and
 *            fixed inputs.
 *   workspace / workspace_bytes: device scratch for the split partials
 *            (miattn_decode_workspace_bytes bytes). workspace == NULL uses a
 *            library-owned buffer (see "Library-owned workspaces" above). Not
 *            used when the split count is 1. A caller workspace must not be
 *            in use by another call that may run at the same time.
 * Robustness: seq_lens are clamped to [0, max_pages_per_seq * 16]; a block
 * table entry outside [0, num_pages) makes that page contribute nothing. Such
 * inputs never fault, but their results are unspecified.
 */
int miattn_attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens,
                             int batch, int max_pages_per_seq, int page_size, int num_pages,
                             int num_q_heads, int num_kv_heads, int head_dim, float scale,
                             int num_splits, void* workspace, size_t workspace_bytes,
                             void* o, float* lse, void* stream);

/*
 * miattn_attn_decode_paged_noalloc -- miattn_attn_decode_paged for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. It calls no hipMalloc, hipFree or
 * allocating library routine. The split partials go to a static device
 * buffer of MIATTN_NOALLOC_SCRATCH_BYTES that the library holds on every GPU
 * it runs on until the process ends; its address is looked up once per
 * device, on the first call made there.
 *   Arguments, layouts, split plan, numerics and results are those of
 *   miattn_attn_decode_paged (bitwise the same outputs) without the
 *   workspace pair. A call whose partials would need more than
 *   MIATTN_NOALLOC_SCRATCH_BYTES (miattn_decode_workspace_bytes for the
 *   resolved split count) returns MIATTN_ERR_WORKSPACE and enqueues nothing.
 *   Every call on one GPU uses the same buffer, whatever its stream: calls
 *   that may run at the same time on one GPU (other streams, other threads)
 *   race and give wrong results. Nothing in the buffer needs to start at
 *   zero: each call writes every partial it reads.
 */
#define MIATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
int miattn_attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     int batch, int max_pages_per_seq, int page_size, int num_pages,
                                     int num_q_heads, int num_kv_heads, int head_dim, float scale,
                                     int num_splits, void* o, float* lse, void* stream);

/*
 * miattn_attn_combine -- merge split partials by log-sum-exp weights (the
 * FlashAttention 2 merge of "Why your local LLM feels dumber than it is",
 * section "Backend names expand into four decode algorithms"):
 *     M = max_s LSE_s over non-empty splits, w_s = exp(LSE_s - M),
 *     O = sum_s w_s O_s / sum_s w_s,   LSE = M + ln sum_s w_s,
 * the sums taken in one fixed order (strided groups of splits, then a
 * pairwise fold of the groups), so the result is bitwise repeatable. A split with
 * LSE_s = -inf is empty and skipped; a row whose splits are all empty gives
 * O = 0, LSE = -inf.
 *   partial_o   [rows, num_splits, D] float32 (normalised partial outputs)
 *   partial_lse [rows, num_splits]    float32
 *   o [rows, D] of out_dtype (MIATTN_BF16 or MIATTN_FP32); lse [rows] float32
 *   (may be NULL). D: 1 .. 1024 and a multiple of 4. rows == 0 is a no-op.
 */
int miattn_attn_combine(const float* partial_o, const float* partial_lse, int rows,
                        int num_splits, int head_dim, void* o, float* lse, int out_dtype,
                        void* stream);

/* Bytes of workspace miattn_attn_decode_paged needs for the partials:
 * 0 when num_splits == 1; for num_splits == 0 an upper bound for the
 * library's plan ((256 + batch) groups per query head). */
size_t miattn_decode_workspace_bytes(int batch, int num_q_heads, int head_dim, int num_splits);

/*
 * miattn_attn_decode_paged_numerics -- the same paged split-KV decode with the
 * split records, rounding points and group geometry selectable, so that the
 * decode programs compared in "Why your local LLM feels dumber than it is"
 * (section "Backend names expand into four decode algorithms"; rounding points
 * of "Why the calculation is split into groups") can be run with this
 * library's arithmetic and set against each other and the exact result. It is
 * a numerics-study entry point: miattn_attn_decode_paged is the fast path.
 *
 * numerics = one record kind | optional flags:
 *   MIATTN_RECORD_LSE: each group stores its normalised fp32 partial and
 *       fp32 LSE; log-sum-exp merge (what miattn_attn_decode_paged does).
 *   MIATTN_RECORD_NUMERATOR_F32: fp32 numerator, reference max m_s and
 *       normaliser l_s; merge O = sum num_s e^(m_s-M) / sum l_s e^(m_s-M).
 *   MIATTN_RECORD_NORMALIZED_BF16: the normalised partial rounded to bf16,
 *       m_s, l_s; merge O = sum o_s l_s e^(m_s-M) / sum l_s e^(m_s-M).
 *   MIATTN_RECORD_NUMERATOR_BF16: the numerator rounded to bf16, m_s, l_s;
 *       an ordered running merge over s = 0, 1, ... in which a still-empty
 *       running state gets weight 0 and empty groups are skipped.
 *   MIATTN_NUMERICS_ROUNDED_NORMALIZER: l_s sums the rounded weights that
 *       enter P.V (bf16, or fp16 with the next flag) instead of fp32 ones.
 *   MIATTN_NUMERICS_P_FP16: P is rounded to fp16 instead of bf16 and V is
 *       converted to fp16 for the P.V product; values of V outside fp16's
 *       range (|v| > 65504) overflow, below 2^-14 they lose precision.
 * m_s is the running max the group's weights were taken against (it may lag
 * the group's true max by up to 2^8 in weight), which leaves every merge exact
 * in real arithmetic.
 * tile_pages: 0 = contiguous groups exactly as miattn_attn_decode_paged;
 *   a power of two <= 1024 = tiles of tile_pages pages dealt round robin,
 *   tile j of a sequence to group j mod num_splits (counts above the number
 *   of tiles of the table width are lowered to it).
 * num_splits: as for miattn_attn_decode_paged (0 = library policy); the
 *   records and the merge are used at every count, 1 included.
 * o [batch, Hq, D] of out_dtype (MIATTN_BF16 or MIATTN_FP32, the latter for
 *   the output before its final rounding); lse [batch, Hq] float32 or NULL.
 * workspace: miattn_decode_numerics_workspace_bytes bytes, or NULL for the
 *   library-owned buffer of the stream (shared with its other calls).
 * Other arguments, layouts, limits and errors as for
 * miattn_attn_decode_paged; unknown numerics bits or a bad tile_pages give
 * MIATTN_ERR_UNSUPPORTED.
 */
#define MIATTN_RECORD_LSE                   0
#define MIATTN_RECORD_NUMERATOR_F32         1
#define MIATTN_RECORD_NORMALIZED_BF16       2
#define MIATTN_RECORD_NUMERATOR_BF16        3
#define MIATTN_NUMERICS_ROUNDED_NORMALIZER  4
#define MIATTN_NUMERICS_P_FP16              8
int miattn_attn_decode_paged_numerics(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      int batch, int max_pages_per_seq, int page_size, int num_pages,
                                      int num_q_heads, int num_kv_heads, int head_dim, float scale,
                                      int num_splits, int numerics, int tile_pages, void* workspace,
                                      size_t workspace_bytes, void* o, int out_dtype, float* lse,
                                      void* stream);

/* Bytes of workspace miattn_attn_decode_paged_numerics needs:
 * batch * Hq * num_splits * (head_dim + 2) floats, rounded up to 256. */
size_t miattn_decode_numerics_workspace_bytes(int batch, int num_q_heads, int head_dim, int num_splits);

/*
 * miattn_attn_bwd -- gradients of attention (the operation of miattn_attn_fwd,
 * bf16) with respect to q, k and v for an upstream gradient dout, by
 * recomputation: the scores are rebuilt tile by tile from q, k and the
 * forward's log-sum-exp, as the backward pass of "Why your local LLM feels
 * dumber than it is" (its ELI5) describes, instead of being stored:
 *     P = exp(scale q.k - LSE),  dV = P^T dO,  dP = dO V^T,
 *     dS = P (dP - rowsum(dO o O)),  dQ = scale dS K,  dK = scale dS^T Q.
 * With GQA, dK/dV of a kv head sum the contributions of all its query heads.
 *   q, o, dout [total_tokens, Hq, D] bf16; k, v [total_tokens, Hkv, D] bf16;
 *   lse [Hq, total_tokens] float32 as written by miattn_attn_fwd for the same
 *   q, k, v (o likewise); cu_seqlens, num_seqs, max_seqlen, scale, causal as
 *   for miattn_attn_fwd.
 *   dq [total_tokens, Hq, D], dk, dv [total_tokens, Hkv, D] bf16 (written).
 *   head_dim 64, 128 or 256 (MIATTN_ERR_UNSUPPORTED otherwise); any Hq/Hkv.
 *   workspace: miattn_attn_bwd_workspace_bytes bytes of device scratch (row
 *   terms and fp16 copies of the inputs), or NULL for the library-owned
 *   buffer of the stream. Inputs must lie inside fp16's range (|x| <= 65504): the products
 *   run on fp16 operands, to which bf16 values inside that range convert
 *   exactly.
 * Deterministic: fixed reduction orders, no atomics; dQ is computed by its own
 * pass over the keys rather than accumulated across workgroups.
 */
int miattn_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                    int total_tokens, int num_q_heads, int num_kv_heads, int head_dim, float scale,
                    int causal, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Bytes of workspace miattn_attn_bwd needs: the fp32 row terms and log2-unit
 * LSE (2 * Hq * (total_tokens + 32..95) floats) and fp16 copies of q, dout, k
 * and v (2 * total_tokens * (Hq + Hkv) * head_dim halves), each rounded up to
 * 256 bytes; 0 for an empty problem. */
size_t miattn_attn_bwd_workspace_bytes(int total_tokens, int num_q_heads, int num_kv_heads, int head_dim);

/* Split count chosen for num_splits == 0: the candidate set and efficiency of
 * miattn_split_heuristic with this library's MI355X capacity (256 compute
 * units, one decode workgroup each), 16-token pages as blocks, work units =
 * batch x kv-head groups of a workgroup, at most 256 splits; the smallest
 * candidate reaching the best efficiency is taken. */
int miattn_decode_pick_splits(int batch, int num_kv_heads, int max_seq_len);

/* The split-count rule described in "Why your local LLM feels dumber than it
 * is", section "Why FlashAttention 2 selects 54, 62, or 87 groups": capacity =
 * cu_count * wg_per_cu; a candidate s scores work_units * s / capacity and
 * efficiency ratio / ceil(ratio); candidates that do not change the blocks per
 * split are skipped; the smallest candidate within 85% of the best efficiency
 * wins; candidates run from 1 to min(max_splits, capacity, blocks).
 * Returns the split count, or MIATTN_ERR_INVALID_ARG for non-positive input. */
int miattn_split_heuristic(int total_tokens, int work_units, int cu_count, int wg_per_cu,
                           int block_tokens, int max_splits);

/* Thread-local description of the last failure ("" if none). */
const char* miattn_last_error(void);
/* Library version: major * 10000 + minor * 100 + patch. */
int miattn_version(void);
/* 1 if HIP device `device` is a gfx950 the kernels were built for, else 0. */
int miattn_device_supported(int device);
/* Free every library-owned workspace on every device, retired ones included.
 * Call it only when no library work is enqueued or running: it frees memory
 * that such work may use (hipFree itself waits for the device). */
void miattn_release(void);

#ifdef __cplusplus
}
#endif
#endif /* MIATTN_H */
