/*
 * attn_varlen.h — C ABI of the MI355X (gfx950) exact-attention library for packed
 * variable-length sequences with grouped-query heads.
 *
 * Sources (page title, section):
 *  [A100]  "[BUG] FA2 vs NATTEN on A100: 3.5-4.8x perf gap; what is the 'flash2
 *          varlen instability' in checks.py?" (cosmos-framework issue), benchmark
 *          script: attention(q, k, v, cumulative_seqlen_Q, cumulative_seqlen_KV,
 *          max_seqlen_Q, max_seqlen_KV); cumulative seqlens are int32 device tensors,
 *          the max seqlens host integers; 32 query heads over 8 KV heads.
 *  [LSE]   "[FA4/B200] return_lse=True makes D64 forward about 19% faster", repro
 *          script, make_call: caller-allocated out and an optional fp32 lse buffer,
 *          with and without the LSE output.
 *  [HD256] "FA4 head_dim=256 B200 Regression Check", Environment: head_dim =
 *          head_dim_v, softmax_scale = head_dim ** -0.5, causal and non-causal.
 *  [GUIDE] FlashAttention repository guide (CLAUDE.md), Public API (varlen entry
 *          point with cu_seqlens_q / cu_seqlens_k; last dimension contiguous,
 *          16-byte aligned), Backward Kernels (preprocess, main, postprocess).
 *
 * Operation (forward). For each packed sequence b with query rows
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key rows [cu_seqlens_k[b],
 * cu_seqlens_k[b+1]), each query head h and its KV head g = h / (n_q_heads /
 * n_kv_heads):
 *     s_ij  = softmax_scale * <q_i, k_j>          (fp32 accumulation of bf16 inputs)
 *     visible(i, j) = !causal || j <= i + Lk - Lq (causal mask aligned bottom-right)
 *     lse_i = ln sum_{visible j} exp(s_ij)
 *     out_i = sum_{visible j} exp(s_ij - lse_i) * v_j
 * A row with no visible key gets out = 0 and lse = -inf.
 *
 * Layouts (all row-major, last dimension unit-stride, no padding):
 *     q, out, dout, dq : bf16 [total_q][n_q_heads][head_dim]
 *     k, v, dk, dv     : bf16 [total_k][n_kv_heads][head_dim]
 *     lse              : fp32 [n_q_heads][total_q]
 *     cu_seqlens_q/_k  : int32 [num_seqs + 1], device memory, cu[0] = 0,
 *                        non-decreasing, cu[num_seqs] = total
 * bf16 is IEEE bfloat16 (1-8-7) stored as 16-bit words; outputs are rounded to
 * nearest-even.
 *
 * Ownership: the caller allocates every buffer (device memory) and keeps it alive
 * until the work on `stream` is done. The library allocates nothing, frees
 * nothing and keeps no pointer after a call returns. A pointer to a tensor with
 * no rows may be NULL: q, out, dout, dq and the LSE of the backward when
 * total_q = 0, and k, v, dk and dv when total_k = 0. A workspace may be NULL
 * when its size is 0. The cu_seqlens arrays are never NULL.
 *
 * Size limits (ATTN_VARLEN_ERR_BAD_SEQLEN otherwise): total_q and total_k below
 * 2^31; within one sequence rows are addressed with 32-bit byte offsets that
 * stay below 2 GiB, tile overruns past the last row included, so
 * (max_seqlen_q + 128) * n_q_heads * head_dim * 2 and (max_seqlen_k + 64) *
 * n_kv_heads * head_dim * 2 must be below 2^31 (e.g. at most 262015 tokens in a
 * sequence with 32 query heads of 128); and the largest launch, (total_q +
 * total_k) / 64 + 2 * num_seqs blocks of 256 threads per query head, must stay
 * below 2^32 threads.
 *
 * Execution: calls are asynchronous on `stream` (a hipStream_t, passed as void*;
 * NULL is the default stream) and never synchronise the host. They run on the
 * calling thread's current HIP device: `stream` and every buffer must belong to
 * it. They are re-entrant and stateless. Identical inputs give bit-identical outputs (no
 * atomics; every reduction runs in a fixed order).
 *
 * Errors: 0 on success, a negative ATTN_VARLEN_ERR_* code otherwise. Every
 * argument check runs before any HIP call, so a rejected call touches no device
 * state. Preconditions on device-resident data (the cu_seqlens contents agree
 * with num_seqs, totals and max seqlens) are not checked: a violation gives
 * undefined results.
 */
#ifndef ATTN_VARLEN_H
#define ATTN_VARLEN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ATTN_VARLEN_OK = 0,
  ATTN_VARLEN_ERR_NULL_POINTER = -1,      /* a required pointer is NULL */
  ATTN_VARLEN_ERR_BAD_HEAD_DIM = -2,      /* head_dim not in {64, 128, 256} */
  ATTN_VARLEN_ERR_BAD_HEADS = -3,         /* heads <= 0 or n_q_heads % n_kv_heads != 0 */
  ATTN_VARLEN_ERR_BAD_SEQLEN = -4,        /* num_seqs < 1, negative totals/max, max > total, or too large */
  ATTN_VARLEN_ERR_MISALIGNED = -5,        /* a tensor pointer is not 16-byte aligned (lse: 4-byte) */
  ATTN_VARLEN_ERR_BAD_SCALE = -6,         /* softmax_scale is not finite */
  ATTN_VARLEN_ERR_WORKSPACE = -7,         /* workspace NULL or smaller than the size its call needs */
  ATTN_VARLEN_ERR_BAD_FLAG = -8,          /* causal not 0 or 1 */
  ATTN_VARLEN_ERR_HIP = -9,               /* the HIP runtime reported an error at launch */
  ATTN_VARLEN_ERR_BAD_SPLITS = -10,       /* num_splits outside [1, ATTN_VARLEN_MAX_SPLITS] */
  ATTN_VARLEN_ERR_SCRATCH_TOO_SMALL = -11 /* attn_varlen_bwd_noalloc: the problem's row terms exceed
                                             ATTN_VARLEN_NOALLOC_SCRATCH_BYTES */
};

#define ATTN_VARLEN_MAX_SPLITS 64

/*
 * Forward pass. [A100] benchmark script `call`; [LSE] make_call (out=, lse=,
 * return_lse); [GUIDE] Public API.
 *   q, k, v            inputs (layouts above)
 *   cu_seqlens_q/_k    packing of queries / keys, device int32 [num_seqs + 1]
 *   num_seqs           number of packed sequences (>= 1); zero-length sequences are legal
 *   total_q, total_k   cu_seqlens_q[num_seqs], cu_seqlens_k[num_seqs]
 *   max_seqlen_q/_k    upper bounds of the per-sequence lengths (host values)
 *   n_q_heads, n_kv_heads, head_dim   head counts (n_q_heads % n_kv_heads == 0) and D
 *   softmax_scale      multiplies the fp32 dot products (any finite value)
 *   causal             0 or 1
 *   out                output, bf16 [total_q][n_q_heads][head_dim]
 *   lse                optional fp32 [n_q_heads][total_q]; NULL skips the LSE write
 */
int attn_varlen_fwd(const void* q, const void* k, const void* v,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                    int32_t num_seqs, int64_t total_q, int64_t total_k,
                    int32_t max_seqlen_q, int32_t max_seqlen_k,
                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                    float softmax_scale, int32_t causal,
                    void* out, float* lse, void* stream);

/*
 * Forward pass with local (sliding-window) attention ([GUIDE] Public API:
 * window_size_left / window_size_right; Core Abstractions: the local mask).
 * Arguments as attn_varlen_fwd, plus:
 *   window_left, window_right  key j of a sequence is visible to query i when
 *                       i + (Lk - Lq) - window_left <= j <= i + (Lk - Lq) + window_right;
 *                       a negative value leaves that side unbounded. causal = 1
 *                       intersects this with j <= i + (Lk - Lq), i.e. a right bound
 *                       of 0. (-1, -1) with causal = 0 is full attention; rows
 *                       that see no key get out = 0 and lse = -inf. A side at
 *                       least total_k (left) or total_q (right) bounds no row
 *                       and is taken as unbounded (bit-identical results).
 *                       No error codes beyond those of attn_varlen_fwd.
 * attn_varlen_fwd is this call with window_left = window_right = -1.
 */
int attn_varlen_fwd_window(const void* q, const void* k, const void* v,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int32_t num_seqs, int64_t total_q, int64_t total_k,
                           int32_t max_seqlen_q, int32_t max_seqlen_k,
                           int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                           float softmax_scale, int32_t causal,
                           int32_t window_left, int32_t window_right,
                           void* out, float* lse, void* stream);

/*
 * Split-KV forward ([GUIDE] Public API: num_splits; Forward Kernels: the
 * combine kernel that merges partial outputs and LSEs). The visible key tiles
 * of every (query block, query head) item are cut into num_splits contiguous
 * chunks computed by separate workgroups; each writes its partial output and
 * row log-sum-exp to the workspace, and a second kernel merges them in chunk
 * order. The result is the forward of attn_varlen_fwd_window (same arguments,
 * same outputs), up to rounding; it pays off when there are too few items to
 * fill the GPU (short query chunks against long keys).
 *   num_splits         1 .. ATTN_VARLEN_MAX_SPLITS; 1 runs the one-pass kernel
 *                      (bit-identical to attn_varlen_fwd_window, workspace unused)
 *   workspace          device scratch of at least
 *                      attn_varlen_fwd_splitkv_workspace_size() bytes, 16-byte
 *                      aligned (may be NULL when num_splits = 1); contents on
 *                      entry are ignored
 * Errors: those of attn_varlen_fwd_window, ATTN_VARLEN_ERR_BAD_SPLITS,
 * ATTN_VARLEN_ERR_WORKSPACE. Deterministic: fixed chunking and merge order.
 */
int attn_varlen_fwd_splitkv(const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            int32_t num_seqs, int64_t total_q, int64_t total_k,
                            int32_t max_seqlen_q, int32_t max_seqlen_k,
                            int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                            float softmax_scale, int32_t causal,
                            int32_t window_left, int32_t window_right, int32_t num_splits,
                            void* out, float* lse, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * Forward with persistent, varlen-aware scheduling ([GUIDE] Core
 * Abstractions: the persistent tile scheduler). Same arguments, outputs and
 * results as attn_varlen_fwd_window (bit-identical: each work item runs the
 * same code); only the assignment of work items to workgroups differs. The
 * kernel launches as many workgroups as the GPU holds at once; they take the
 * (query block, query head) items, longest first, from eight per-XCD queues
 * (their own XCD's first, then the others), so that faster XCDs take more work.
 *   sched              device scratch of ATTN_VARLEN_SCHED_BYTES bytes, 4-byte
 *                      aligned, all zero before its first use; every call
 *                      leaves it zero again. Calls that share one sched buffer
 *                      must not run concurrently (stream-ordered use is fine).
 * Errors: those of attn_varlen_fwd_window; ATTN_VARLEN_ERR_WORKSPACE for a NULL
 * sched, ATTN_VARLEN_ERR_MISALIGNED for a misaligned one.
 */
#define ATTN_VARLEN_SCHED_BYTES 64
int attn_varlen_fwd_persistent(const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t num_seqs, int64_t total_q, int64_t total_k,
                               int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                               float softmax_scale, int32_t causal,
                               int32_t window_left, int32_t window_right,
                               void* out, float* lse, void* sched, void* stream);

/*
 * Workspace bytes of attn_varlen_fwd_splitkv: fp32 partial outputs
 * [num_splits][total_q][n_q_heads][head_dim] and fp32 row sums
 * [num_splits][2][n_q_heads][total_q], each rounded up to 256 bytes; 0 when
 * num_splits <= 1 or for negative sizes / non-positive heads.
 */
size_t attn_varlen_fwd_splitkv_workspace_size(int64_t total_q, int32_t n_q_heads, int32_t head_dim,
                                              int32_t num_splits);

/*
 * A split count for these sizes (host-only, no device access): the number of
 * chunks that best fills the GPU's concurrent workgroup slots with the
 * forward's (query block, head) items, keeping every chunk at least four key
 * tiles long; 1 when the items already fill the GPU. Returns a negative
 * ATTN_VARLEN_ERR_* code for bad sizes or heads.
 */
int32_t attn_varlen_fwd_num_splits(int32_t num_seqs, int64_t total_q, int32_t max_seqlen_q,
                                   int32_t max_seqlen_k, int32_t n_q_heads, int32_t n_kv_heads,
                                   int32_t head_dim);

/*
 * Device-side check of the packing arrays, which every call takes as a
 * precondition (the host-side checks only see the sizes): cu_seqlens_q[0] and
 * cu_seqlens_k[0] are 0, both arrays are non-decreasing, their last entries are
 * total_q and total_k, and no sequence is longer than max_seqlen_q /
 * max_seqlen_k. Asynchronous on `stream`: writes to `result` (one device int32)
 * a bit mask, 0 when the arrays are valid, else an OR of
 *   ATTN_VARLEN_SEQLEN_BAD_START (1)  a first entry is not 0
 *   ATTN_VARLEN_SEQLEN_DECREASING (2) an entry is smaller than the one before
 *   ATTN_VARLEN_SEQLEN_BAD_TOTAL (4)  a last entry differs from the total
 *   ATTN_VARLEN_SEQLEN_OVER_MAX (8)   a sequence is longer than its max_seqlen
 * Errors: ATTN_VARLEN_ERR_NULL_POINTER, ATTN_VARLEN_ERR_BAD_SEQLEN (num_seqs < 1,
 * negative sizes), ATTN_VARLEN_ERR_MISALIGNED (result not 4-byte aligned),
 * ATTN_VARLEN_ERR_HIP. The Python binding runs it before each call when the
 * environment variable ATTN_VARLEN_VALIDATE is 1 and raises on a non-zero mask.
 */
#define ATTN_VARLEN_SEQLEN_BAD_START 1
#define ATTN_VARLEN_SEQLEN_DECREASING 2
#define ATTN_VARLEN_SEQLEN_BAD_TOTAL 4
#define ATTN_VARLEN_SEQLEN_OVER_MAX 8
int attn_varlen_validate_seqlens(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
                                 int64_t total_q, int64_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                 int32_t* result, void* stream);

/*
 * Bytes of device workspace attn_varlen_bwd needs for these sizes. It holds the
 * fp32 row term Delta_i = sum_d dout_id * out_id per query row and head ([GUIDE]
 * Backward Kernels: the preprocess kernel) and the LSE in base 2, each
 * [n_q_heads][total_q]. At head_dim 256 with few key blocks per KV head, it
 * also holds fp32 partial dK / dV sums, [s][total_k][n_kv_heads][256] each,
 * where s divides n_q_heads / n_kv_heads. Each part is rounded up to 256 bytes.
 * Returns 0 for negative sizes or non-positive head counts.
 */
size_t attn_varlen_bwd_workspace_size(int32_t num_seqs, int64_t total_q, int64_t total_k,
                                      int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim);

/*
 * Bytes of device workspace attn_varlen_bwd_stored_ds needs, or 0 where that
 * call is not available (head dim 256, an empty problem, or one sequence's rows
 * of its dS buffer spanning 2 GiB or more): attn_varlen_bwd_workspace_size()
 * plus n_q_heads * total_k * (64 + 128 * ceil(max_seqlen_q / 128)) * 2 bytes,
 * rounded up to 256.
 */
size_t attn_varlen_bwd_ds_workspace_size(int32_t num_seqs, int64_t total_q, int64_t total_k,
                                         int32_t max_seqlen_q, int32_t max_seqlen_k,
                                         int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim);

/*
 * Backward pass: gradients of sum(dout * out) with respect to q, k, v for the
 * forward defined above ([A100] benchmark script `fb`: forward then
 * out.backward(dout); [GUIDE] Backward Kernels). Arguments up to `causal` are
 * those of the forward call that produced `out` and `lse`.
 *   dout, out          bf16 [total_q][n_q_heads][head_dim]
 *   lse                fp32 [n_q_heads][total_q] from the forward (required)
 *   dq                 bf16 [total_q][n_q_heads][head_dim]     (written)
 *   dk, dv             bf16 [total_k][n_kv_heads][head_dim]    (written; summed over
 *                      the query heads of each KV head's group)
 *   workspace          device scratch of at least attn_varlen_bwd_workspace_size()
 *                      bytes, 16-byte aligned; contents on entry are ignored
 * Every element of dq, dk, dv is written (keys no query can see get zero).
 */
int attn_varlen_bwd(const void* q, const void* k, const void* v,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                    int32_t num_seqs, int64_t total_q, int64_t total_k,
                    int32_t max_seqlen_q, int32_t max_seqlen_k,
                    int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                    float softmax_scale, int32_t causal,
                    const void* dout, const void* out, const float* lse,
                    void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass of attn_varlen_fwd_window (same window arguments; the same
 * workspace size as attn_varlen_bwd). attn_varlen_bwd is this call with
 * window_left = window_right = -1.
 */
int attn_varlen_bwd_window(const void* q, const void* k, const void* v,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int32_t num_seqs, int64_t total_q, int64_t total_k,
                           int32_t max_seqlen_q, int32_t max_seqlen_k,
                           int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                           float softmax_scale, int32_t causal,
                           int32_t window_left, int32_t window_right,
                           const void* dout, const void* out, const float* lse,
                           void* dq, void* dk, void* dv,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward with dS stored for dQ instead of recomputed (head dims 64 / 128).
 * The main kernel ([GUIDE] Backward Kernels) forms dS = P * (dP - Delta) for
 * dK; here it also writes dS in bf16 (the value its dK product uses) to a
 * buffer in the workspace, one row per (query head, key) of max_seqlen_q
 * rounded up to 128, plus 64, columns, and the dQ kernel forms dQ =
 * softmax_scale * dS K from it: one product per visible key tile instead of
 * recomputing S, P and dP. The trade is two bf16 passes over every visible
 * (query, key, head) through HBM for 4 * head_dim flop per pair; on MI355X the
 * recomputing attn_varlen_bwd_window is faster at every measured shape (packed
 * 16K documents, 4K and 16K sequences, head dims 64 and 128), so this call is
 * an alternative, not the default. Same arguments and results as
 * attn_varlen_bwd_window (deterministic; dQ and dK can differ from it by
 * rounding: the row term Delta is summed in another order), plus:
 *   workspace          at least attn_varlen_bwd_ds_workspace_size() bytes, 16-byte aligned
 * Errors: those of attn_varlen_bwd_window; ATTN_VARLEN_ERR_BAD_HEAD_DIM for head
 * dim 256; ATTN_VARLEN_ERR_BAD_SEQLEN when the size call returns 0 for a
 * non-empty problem.
 */
int attn_varlen_bwd_stored_ds(const void* q, const void* k, const void* v,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t num_seqs, int64_t total_q, int64_t total_k,
                              int32_t max_seqlen_q, int32_t max_seqlen_k,
                              int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                              float softmax_scale, int32_t causal,
                              int32_t window_left, int32_t window_right,
                              const void* dout, const void* out, const float* lse,
                              void* dq, void* dk, void* dv,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free backward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). The same computation, arguments and results as attn_varlen_bwd
 * (the same kernels; bit-identical whenever the scratch holds the workspace
 * attn_varlen_bwd_workspace_size gives), without the workspace arguments: the
 * workspace lives in a device array inside the library,
 * ATTN_VARLEN_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, which each GPU the
 * library runs on holds until the process ends. The call allocates nothing and
 * frees nothing; the caller still passes every input and output.
 *   Limit: the row terms take 8 bytes per (query row, query head); problems
 *   whose row terms exceed the scratch (more than 4M query row-heads, e.g. 32
 *   heads x 128K tokens) are rejected with ATTN_VARLEN_ERR_SCRATCH_TOO_SMALL
 *   before any HIP call. With few key blocks per KV head the dK / dV work splits
 *   a group's query heads and keeps fp32 partial sums in the workspace; here it
 *   uses as many splits as the scratch holds, and where that is fewer than
 *   attn_varlen_bwd uses, dK and dV differ from its by fp32 summation order
 *   (the result stays deterministic).
 *   Sharing: every call on one GPU uses that GPU's one scratch array, which keeps
 *   the last call's contents (nothing in it needs to start at zero). Calls on
 *   one GPU must therefore not overlap: calls on different streams, or from
 *   several host threads, that may run at the same time race on the scratch.
 *   Calls ordered on one stream are fine.
 * Errors: those of attn_varlen_bwd except ATTN_VARLEN_ERR_WORKSPACE, plus
 * ATTN_VARLEN_ERR_SCRATCH_TOO_SMALL, and ATTN_VARLEN_ERR_HIP if the scratch's
 * device address cannot be looked up.
 */
#define ATTN_VARLEN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int attn_varlen_bwd_noalloc(const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            int32_t num_seqs, int64_t total_q, int64_t total_k,
                            int32_t max_seqlen_q, int32_t max_seqlen_k,
                            int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                            float softmax_scale, int32_t causal,
                            const void* dout, const void* out, const float* lse,
                            void* dq, void* dk, void* dv, void* stream);

/* Static description of an error code. Never NULL. */
const char* attn_varlen_error_string(int code);

/* Library ABI version: (major << 16) | minor. */
int attn_varlen_version(void);

/*
 * Work-list inspection (host, no GPU needed): the order in which the forward
 * visits query blocks. Query blocks of `block_m` rows are ranked by descending
 * block index (longest causal work first), ties by ascending sequence. Writes the
 * sequence index and block index of rank r to seq_out[r], block_out[r] for
 * r < min(capacity, count) and returns count, or a negative error code.
 * cu_seqlens_q_host is a host array of num_seqs + 1 entries.
 */
int64_t attn_varlen_schedule_host(const int32_t* cu_seqlens_q_host, int32_t num_seqs, int32_t block_m,
                                  int32_t* seq_out, int32_t* block_out, int64_t capacity);

/*
 * The same ranking computed by the device code path the kernels use, for
 * `count` ranks starting at 0: seq_out / block_out are device int32 [count];
 * ranks beyond the number of blocks get -1. Asynchronous on `stream`.
 */
int attn_varlen_schedule_device(const int32_t* cu_seqlens_q, int32_t num_seqs, int32_t max_seqlen_q,
                                int32_t block_m, int32_t* seq_out, int32_t* block_out, int32_t count,
                                void* stream);

/*
 * Tile plan inspection (host, no GPU needed): which tiles a kernel visits for
 * one work item of a one-sequence batch, and which of them it runs without a
 * mask ([GUIDE] Core Abstractions: the block-info helper that gives the range
 * of key blocks a query block meets under causal and local masks). Visiting
 * every tile that holds a visible (query, key) pair and masking every tile
 * that holds a hidden one is what makes the kernels exact; the tests check
 * both by enumerating every pair of small sequences.
 *   kind        ATTN_VARLEN_PLAN_FWD  query block `block` of the forward kernel
 *               ATTN_VARLEN_PLAN_DQ   query block `block` of the dQ kernel
 *               ATTN_VARLEN_PLAN_DKDV key block `block` of the dK / dV kernel
 *               FWD or DQ may be or-ed with ATTN_VARLEN_PLAN_GROUP2 or
 *               ATTN_VARLEN_PLAN_GROUP4: the blocks these kernels take when the
 *               KV group size (n_q_heads / n_kv_heads) is a multiple of 2 but
 *               not of 4, or a multiple of 4. A workgroup then covers 2 or 4
 *               query heads of one KV group and 64 or 32 rows of each; without
 *               a flag it covers one head and 128 rows. (The dQ kernel that
 *               reads stored dS always takes one head and 128 rows.)
 *   head_dim    64, 128 or 256 (tile shapes depend on it)
 *   seqlen_q, seqlen_k, causal, window_left, window_right
 *               the sequence and its mask, as in attn_varlen_fwd_window
 *   plan        int32[8], written:
 *               [0] first row (query blocks; may be negative: the blocks are
 *                   aligned toward the sequence end) or first key (key blocks)
 *               [1] rows (query blocks) or keys (key blocks) per block
 *               [2] keys per key tile (FWD, DQ) or rows per query step (DKDV)
 *               [3], [4] the tiles visited, [lo, hi)
 *               [5], [6] the tiles run without a mask, [lo, hi) (empty if hi <= lo)
 *               [7] FWD with a left window bound: the left-edge tiles [lo, lo + [7])
 *                   whose scores are masked but whose probabilities take the
 *                   unmasked path; 0 otherwise
 *               A tile index t covers keys (or query rows) [t * plan[2], (t + 1) * plan[2]).
 * Errors: ATTN_VARLEN_ERR_NULL_POINTER, ATTN_VARLEN_ERR_BAD_HEAD_DIM,
 * ATTN_VARLEN_ERR_BAD_FLAG (causal or kind), ATTN_VARLEN_ERR_BAD_SEQLEN
 * (negative lengths, block out of range).
 */
#define ATTN_VARLEN_PLAN_FWD 0
#define ATTN_VARLEN_PLAN_DQ 1
#define ATTN_VARLEN_PLAN_DKDV 2
#define ATTN_VARLEN_PLAN_GROUP2 0x10
#define ATTN_VARLEN_PLAN_GROUP4 0x20
int attn_varlen_tile_plan_host(int32_t kind, int32_t head_dim, int32_t seqlen_q, int32_t seqlen_k, int32_t causal,
                               int32_t window_left, int32_t window_right, int32_t block, int32_t* plan);

/*
 * The forward's FMA-pipe exponential, evaluated on the host for testing
 * ([HD256] Observations: exp2 emulation on FMA units; [GUIDE] Other Components,
 * fast_math): y[i] = 2^x[i] by range reduction x = n + f (n = rint(x)) and a
 * degree-3 minimax polynomial for 2^f, relative error <= 7.5e-5 plus float32
 * rounding for x >= -125, exactly 0 below (and for -inf). The forward kernel
 * uses it for every K-th score of an unmasked tile when the library is built
 * with AV_EXP2_EMU = K (0, the default: the hardware exponential only).
 * Returns K (>= 0), or ATTN_VARLEN_ERR_BAD_SEQLEN (n < 0) /
 * ATTN_VARLEN_ERR_NULL_POINTER.
 */
int attn_varlen_exp2_fma_host(const float* x, float* y, int64_t n);

/*
 * Per-launch timing, for benchmarks. While enabled, every kernel the library
 * launches is bracketed by two HIP events recorded on the launch's stream (the
 * events belong to the library and are reused). attn_varlen_profile_enable(1)
 * starts a new session (drops earlier records); (0) stops recording. Records
 * beyond 65536 per session are dropped. Not meant for concurrent use from
 * several host threads.
 *   attn_varlen_profile_count   number of launches recorded in the session
 *   attn_varlen_profile_get     kernel name (copied, NUL-terminated, truncated to
 *                               name_capacity) and its duration in ms; waits for
 *                               the launch to finish. Returns
 *                               ATTN_VARLEN_ERR_BAD_SEQLEN for an index out of
 *                               range, ATTN_VARLEN_ERR_HIP if the events fail.
 */
int attn_varlen_profile_enable(int enable);
int attn_varlen_profile_count(void);
int attn_varlen_profile_get(int index, char* name, int name_capacity, float* ms);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_VARLEN_H */
