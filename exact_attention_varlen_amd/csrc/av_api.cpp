// av_api.cpp — the C ABI declared in include/attn_varlen.h: argument checks
// (all before any HIP call) and dispatch to the kernel launchers.
#include "../../include/attn_varlen.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "av_exp2.h"
#include "av_launch.h"
#include "av_sched.h"

namespace {

constexpr int kVersionMajor = 1;
constexpr int kVersionMinor = 8;
constexpr int64_t kMaxGridThreads = (int64_t)1 << 32;  // grid x block must stay below 2^32 work-items

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_common(const void* q, const void* k, const void* v, const int32_t* cu_q, const int32_t* cu_k,
                 int32_t num_seqs, int64_t total_q, int64_t total_k, int32_t max_q, int32_t max_k, int32_t Hq,
                 int32_t Hkv, int32_t D, float scale, int32_t causal) {
  // data pointers may be NULL when their tensors are empty (no rows)
  if (!cu_q || !cu_k) return ATTN_VARLEN_ERR_NULL_POINTER;
  if ((total_q > 0 && !q) || (total_k > 0 && (!k || !v))) return ATTN_VARLEN_ERR_NULL_POINTER;
  if (D != 64 && D != 128 && D != 256) return ATTN_VARLEN_ERR_BAD_HEAD_DIM;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return ATTN_VARLEN_ERR_BAD_HEADS;
  if (num_seqs < 1 || total_q < 0 || total_k < 0 || max_q < 0 || max_k < 0) return ATTN_VARLEN_ERR_BAD_SEQLEN;
  if (max_q > total_q || max_k > total_k) return ATTN_VARLEN_ERR_BAD_SEQLEN;
  if (total_q > INT32_MAX || total_k > INT32_MAX) return ATTN_VARLEN_ERR_BAD_SEQLEN;
  // the largest grid any kernel launches (query or key blocks of 64 rows, times
  // the query heads, 256 threads each) must stay below 2^32 work-items
  const int64_t blocks = (total_q + total_k) / 64 + 2 * (int64_t)num_seqs;
  if (blocks * (int64_t)Hq * 256 >= kMaxGridThreads) return ATTN_VARLEN_ERR_BAD_SEQLEN;
  // Rows are addressed with 32-bit buffer offsets relative to a sequence's first
  // row, and every offset a kernel forms must stay below 2 GiB, including those
  // of the rows past the sequence's end that a tile's copy covers (they read as
  // zero): K / V tiles run at most 63 rows past the last key, the dK / dV
  // kernel's query steps (Q, dO) at most 127 rows past the last query.
  if ((int64_t)(max_k + 64) * Hkv * D * 2 >= ((int64_t)1 << 31)) return ATTN_VARLEN_ERR_BAD_SEQLEN;
  if ((int64_t)(max_q + 128) * Hq * D * 2 >= ((int64_t)1 << 31)) return ATTN_VARLEN_ERR_BAD_SEQLEN;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16)) return ATTN_VARLEN_ERR_MISALIGNED;
  if (!aligned(cu_q, 4) || !aligned(cu_k, 4)) return ATTN_VARLEN_ERR_MISALIGNED;
  if (!std::isfinite(scale)) return ATTN_VARLEN_ERR_BAD_SCALE;
  if (causal != 0 && causal != 1) return ATTN_VARLEN_ERR_BAD_FLAG;
  return ATTN_VARLEN_OK;
}

av::FwdArgs make_fwd_args(const void* q, const void* k, const void* v, const int32_t* cu_q, const int32_t* cu_k,
                          int32_t num_seqs, int64_t total_q, int64_t total_k, int32_t max_q, int32_t max_k,
                          int32_t Hq, int32_t Hkv, int32_t D, float scale, int32_t causal, int32_t window_left,
                          int32_t window_right, void* stream) {
  av::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.total_k = total_k;
  a.max_q = max_q;
  a.max_k = max_k;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.scale = scale;
  a.causal = causal;
  // A side wider than any sequence bounds nothing: a left bound >= total_k puts
  // every row's first key below 0, a right bound >= total_q every row's last key
  // past Lk - 1. Such sides become unbounded, so they take the kernels of the
  // plain problem and no per-key arithmetic can overflow.
  a.window_left = (window_left < 0 || window_left >= total_k) ? -1 : window_left;
  a.window_right = (window_right < 0 || window_right >= total_q) ? -1 : window_right;
  a.out = nullptr;
  a.lse = nullptr;
  a.stream = stream;
  return a;
}

int bwd_checked(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                const int32_t* cu_seqlens_k, int32_t num_seqs, int64_t total_q, int64_t total_k,
                int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t n_q_heads, int32_t n_kv_heads,
                int32_t head_dim, float softmax_scale, int32_t causal, int32_t window_left, int32_t window_right,
                const void* dout, const void* out, const float* lse, void* dq, void* dk, void* dv,
                void* workspace, size_t workspace_bytes, bool static_scratch, bool stored_ds, void* stream) {
  int rc = check_common(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q, max_seqlen_k,
                        n_q_heads, n_kv_heads, head_dim, softmax_scale, causal);
  if (rc != ATTN_VARLEN_OK) return rc;
  if ((total_q > 0 && (!dout || !out || !lse || !dq)) || (total_k > 0 && (!dk || !dv)))
    return ATTN_VARLEN_ERR_NULL_POINTER;
  if (!aligned(dout, 16) || !aligned(out, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4))
    return ATTN_VARLEN_ERR_MISALIGNED;
  const size_t need = av::bwd_workspace_bytes(total_q, total_k, n_q_heads, n_kv_heads, head_dim);
  if (stored_ds) {
    // the stored-dS dQ: head dims 64 / 128 and a dS buffer within 32-bit offsets
    if (head_dim > 128) return ATTN_VARLEN_ERR_BAD_HEAD_DIM;
    if (total_q > 0 && total_k > 0) {
      const size_t need_ds = av::bwd_ds_workspace_bytes(total_q, total_k, max_seqlen_q, max_seqlen_k, n_q_heads,
                                                        n_kv_heads, head_dim);
      if (need_ds == 0) return ATTN_VARLEN_ERR_BAD_SEQLEN;
      if (!workspace || workspace_bytes < need_ds) return ATTN_VARLEN_ERR_WORKSPACE;
    } else {
      stored_ds = false;  // nothing to store: the plain path handles empty problems
    }
  }
  if (static_scratch) {
    // the scratch must hold the workspace without dK / dV head splits; the
    // backward then runs with as many splits as it holds
    if (av::bwd_min_workspace_bytes(total_q, total_k, n_q_heads, n_kv_heads, head_dim) >
        av::noalloc_scratch_bytes())
      return ATTN_VARLEN_ERR_SCRATCH_TOO_SMALL;
  } else {
    if (need > 0 && (!workspace || workspace_bytes < need)) return ATTN_VARLEN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return ATTN_VARLEN_ERR_MISALIGNED;
  }
  if (total_q == 0 && total_k == 0) return ATTN_VARLEN_OK;
  if (static_scratch && need > 0) {
    if (av::noalloc_scratch(&workspace) != hipSuccess) return ATTN_VARLEN_ERR_HIP;
  }
  av::BwdArgs a;
  a.f = make_fwd_args(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q, max_seqlen_k,
                      n_q_heads, n_kv_heads, head_dim, softmax_scale, causal, window_left, window_right, stream);
  a.dout = dout;
  a.out = out;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = static_cast<float*>(workspace);
  a.ds = stored_ds ? static_cast<char*>(workspace) + need : nullptr;
  a.ds_pitch = stored_ds ? av::bwd_ds_pitch(max_seqlen_q) : 0;
  a.ws_bytes = static_scratch ? av::noalloc_scratch_bytes() : workspace_bytes;
  return av::launch_bwd(a) == hipSuccess ? ATTN_VARLEN_OK : ATTN_VARLEN_ERR_HIP;
}

}  // namespace

extern "C" {

int attn_varlen_fwd_window(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                           const int32_t* cu_seqlens_k, int32_t num_seqs, int64_t total_q, int64_t total_k,
                           int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t n_q_heads, int32_t n_kv_heads,
                           int32_t head_dim, float softmax_scale, int32_t causal, int32_t window_left,
                           int32_t window_right, void* out, float* lse, void* stream) {
  int rc = check_common(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q, max_seqlen_k,
                        n_q_heads, n_kv_heads, head_dim, softmax_scale, causal);
  if (rc != ATTN_VARLEN_OK) return rc;
  if (total_q > 0 && !out) return ATTN_VARLEN_ERR_NULL_POINTER;
  if (!aligned(out, 16) || (lse && !aligned(lse, 4))) return ATTN_VARLEN_ERR_MISALIGNED;
  if (total_q == 0) return ATTN_VARLEN_OK;
  av::FwdArgs a = make_fwd_args(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q,
                                max_seqlen_k, n_q_heads, n_kv_heads, head_dim, softmax_scale, causal, window_left,
                                window_right, stream);
  a.out = out;
  a.lse = lse;
  return av::launch_fwd(a) == hipSuccess ? ATTN_VARLEN_OK : ATTN_VARLEN_ERR_HIP;
}

int attn_varlen_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                    const int32_t* cu_seqlens_k, int32_t num_seqs, int64_t total_q, int64_t total_k,
                    int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t n_q_heads, int32_t n_kv_heads,
                    int32_t head_dim, float softmax_scale, int32_t causal, void* out, float* lse, void* stream) {
  return attn_varlen_fwd_window(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q,
                                max_seqlen_k, n_q_heads, n_kv_heads, head_dim, softmax_scale, causal, -1, -1, out,
                                lse, stream);
}

int attn_varlen_fwd_splitkv(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int32_t num_seqs, int64_t total_q, int64_t total_k,
                            int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t n_q_heads, int32_t n_kv_heads,
                            int32_t head_dim, float softmax_scale, int32_t causal, int32_t window_left,
                            int32_t window_right, int32_t num_splits, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  int rc = check_common(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q, max_seqlen_k,
                        n_q_heads, n_kv_heads, head_dim, softmax_scale, causal);
  if (rc != ATTN_VARLEN_OK) return rc;
  if (total_q > 0 && !out) return ATTN_VARLEN_ERR_NULL_POINTER;
  if (!aligned(out, 16) || (lse && !aligned(lse, 4))) return ATTN_VARLEN_ERR_MISALIGNED;
  if (num_splits < 1 || num_splits > ATTN_VARLEN_MAX_SPLITS) return ATTN_VARLEN_ERR_BAD_SPLITS;
  // the split grid multiplies the forward's (query block x head) units by num_splits
  if ((total_q / 128 + (int64_t)num_seqs) * n_q_heads * num_splits * 256 >= kMaxGridThreads)
    return ATTN_VARLEN_ERR_BAD_SEQLEN;
  const size_t need = av::split_workspace_bytes(total_q, n_q_heads, head_dim, num_splits);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return ATTN_VARLEN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return ATTN_VARLEN_ERR_MISALIGNED;
  }
  if (total_q == 0) return ATTN_VARLEN_OK;
  av::FwdArgs a = make_fwd_args(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q,
                                max_seqlen_k, n_q_heads, n_kv_heads, head_dim, softmax_scale, causal, window_left,
                                window_right, stream);
  a.out = out;
  a.lse = lse;
  return av::launch_fwd_split(a, num_splits, workspace) == hipSuccess ? ATTN_VARLEN_OK : ATTN_VARLEN_ERR_HIP;
}

int attn_varlen_fwd_persistent(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k, int32_t num_seqs, int64_t total_q, int64_t total_k,
                               int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t n_q_heads, int32_t n_kv_heads,
                               int32_t head_dim, float softmax_scale, int32_t causal, int32_t window_left,
                               int32_t window_right, void* out, float* lse, void* sched, void* stream) {
  static_assert(ATTN_VARLEN_SCHED_BYTES >= av::kSchedWords * 4, "scheduler words");
  int rc = check_common(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q, max_seqlen_k,
                        n_q_heads, n_kv_heads, head_dim, softmax_scale, causal);
  if (rc != ATTN_VARLEN_OK) return rc;
  if (total_q > 0 && !out) return ATTN_VARLEN_ERR_NULL_POINTER;
  if (!sched) return ATTN_VARLEN_ERR_WORKSPACE;
  if (!aligned(out, 16) || (lse && !aligned(lse, 4)) || !aligned(sched, 4)) return ATTN_VARLEN_ERR_MISALIGNED;
  if (total_q == 0) return ATTN_VARLEN_OK;
  av::FwdArgs a = make_fwd_args(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q,
                                max_seqlen_k, n_q_heads, n_kv_heads, head_dim, softmax_scale, causal, window_left,
                                window_right, stream);
  a.out = out;
  a.lse = lse;
  return av::launch_fwd_persistent(a, sched) == hipSuccess ? ATTN_VARLEN_OK : ATTN_VARLEN_ERR_HIP;
}

size_t attn_varlen_fwd_splitkv_workspace_size(int64_t total_q, int32_t n_q_heads, int32_t head_dim,
                                              int32_t num_splits) {
  if (total_q < 0 || n_q_heads <= 0 || head_dim <= 0 || num_splits <= 1) return 0;
  return av::split_workspace_bytes(total_q, n_q_heads, head_dim, num_splits);
}

int32_t attn_varlen_fwd_num_splits(int32_t num_seqs, int64_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                   int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim) {
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return ATTN_VARLEN_ERR_BAD_HEAD_DIM;
  if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0) return ATTN_VARLEN_ERR_BAD_HEADS;
  if (num_seqs < 1 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || max_seqlen_q > total_q)
    return ATTN_VARLEN_ERR_BAD_SEQLEN;
  return av::fwd_num_splits(num_seqs, total_q, max_seqlen_q, max_seqlen_k, n_q_heads, n_kv_heads, head_dim);
}

size_t attn_varlen_bwd_workspace_size(int32_t num_seqs, int64_t total_q, int64_t total_k, int32_t n_q_heads,
                                      int32_t n_kv_heads, int32_t head_dim) {
  (void)num_seqs;
  if (total_q < 0 || total_k < 0 || n_q_heads <= 0 || n_kv_heads <= 0) return 0;
  return av::bwd_workspace_bytes(total_q, total_k, n_q_heads, n_kv_heads, head_dim);
}

size_t attn_varlen_bwd_ds_workspace_size(int32_t num_seqs, int64_t total_q, int64_t total_k, int32_t max_seqlen_q,
                                         int32_t max_seqlen_k, int32_t n_q_heads, int32_t n_kv_heads,
                                         int32_t head_dim) {
  (void)num_seqs;
  if (total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || n_q_heads <= 0 || n_kv_heads <= 0 ||
      n_q_heads % n_kv_heads != 0)
    return 0;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return 0;
  return av::bwd_ds_workspace_bytes(total_q, total_k, max_seqlen_q, max_seqlen_k, n_q_heads, n_kv_heads, head_dim);
}

int attn_varlen_bwd_window(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                           const int32_t* cu_seqlens_k, int32_t num_seqs, int64_t total_q, int64_t total_k,
                           int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t n_q_heads, int32_t n_kv_heads,
                           int32_t head_dim, float softmax_scale, int32_t causal, int32_t window_left,
                           int32_t window_right, const void* dout, const void* out, const float* lse, void* dq,
                           void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_checked(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q, max_seqlen_k,
                     n_q_heads, n_kv_heads, head_dim, softmax_scale, causal, window_left, window_right, dout, out, lse,
                     dq, dk, dv, workspace, workspace_bytes, false, false, stream);
}

int attn_varlen_bwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                    const int32_t* cu_seqlens_k, int32_t num_seqs, int64_t total_q, int64_t total_k,
                    int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t n_q_heads, int32_t n_kv_heads,
                    int32_t head_dim, float softmax_scale, int32_t causal, const void* dout, const void* out,
                    const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return attn_varlen_bwd_window(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q,
                                max_seqlen_k, n_q_heads, n_kv_heads, head_dim, softmax_scale, causal, -1, -1, dout,
                                out, lse, dq, dk, dv, workspace, workspace_bytes, stream);
}

int attn_varlen_bwd_stored_ds(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, int32_t num_seqs, int64_t total_q, int64_t total_k,
                              int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t n_q_heads, int32_t n_kv_heads,
                              int32_t head_dim, float softmax_scale, int32_t causal, int32_t window_left,
                              int32_t window_right, const void* dout, const void* out, const float* lse, void* dq,
                              void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_checked(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q, max_seqlen_k,
                     n_q_heads, n_kv_heads, head_dim, softmax_scale, causal, window_left, window_right, dout, out, lse,
                     dq, dk, dv, workspace, workspace_bytes, false, true, stream);
}

int attn_varlen_bwd_noalloc(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int32_t num_seqs, int64_t total_q, int64_t total_k,
                            int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t n_q_heads, int32_t n_kv_heads,
                            int32_t head_dim, float softmax_scale, int32_t causal, const void* dout,
                            const void* out, const float* lse, void* dq, void* dk, void* dv, void* stream) {
  return bwd_checked(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q, max_seqlen_k,
                     n_q_heads, n_kv_heads, head_dim, softmax_scale, causal, -1, -1, dout, out, lse, dq, dk, dv,
                     nullptr, 0, true, false, stream);
}

int attn_varlen_validate_seqlens(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
                                 int64_t total_q, int64_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                 int32_t* result, void* stream) {
  static_assert(ATTN_VARLEN_SEQLEN_BAD_START == av::kSeqlenBadStart &&
                    ATTN_VARLEN_SEQLEN_DECREASING == av::kSeqlenDecreasing &&
                    ATTN_VARLEN_SEQLEN_BAD_TOTAL == av::kSeqlenBadTotal &&
                    ATTN_VARLEN_SEQLEN_OVER_MAX == av::kSeqlenOverMax,
                "result bits");
  if (!cu_seqlens_q || !cu_seqlens_k || !result) return ATTN_VARLEN_ERR_NULL_POINTER;
  if (num_seqs < 1 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return ATTN_VARLEN_ERR_BAD_SEQLEN;
  if (!aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4) || !aligned(result, 4))
    return ATTN_VARLEN_ERR_MISALIGNED;
  return av::launch_validate_seqlens(cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q,
                                     max_seqlen_k, result, stream) == hipSuccess
             ? ATTN_VARLEN_OK
             : ATTN_VARLEN_ERR_HIP;
}

const char* attn_varlen_error_string(int code) {
  switch (code) {
    case ATTN_VARLEN_OK: return "success";
    case ATTN_VARLEN_ERR_NULL_POINTER: return "a required pointer is NULL";
    case ATTN_VARLEN_ERR_BAD_HEAD_DIM: return "head_dim must be 64, 128 or 256";
    case ATTN_VARLEN_ERR_BAD_HEADS: return "head counts must be positive with n_q_heads a multiple of n_kv_heads";
    case ATTN_VARLEN_ERR_BAD_SEQLEN: return "bad sequence sizes (num_seqs, totals or max seqlens)";
    case ATTN_VARLEN_ERR_MISALIGNED: return "a tensor pointer is misaligned (16 bytes; lse 4 bytes)";
    case ATTN_VARLEN_ERR_BAD_SCALE: return "softmax_scale is not finite";
    case ATTN_VARLEN_ERR_WORKSPACE: return "workspace is NULL or too small";
    case ATTN_VARLEN_ERR_BAD_FLAG: return "causal must be 0 or 1";
    case ATTN_VARLEN_ERR_HIP: return "HIP runtime error at kernel launch";
    case ATTN_VARLEN_ERR_BAD_SPLITS: return "num_splits must be in [1, ATTN_VARLEN_MAX_SPLITS]";
    case ATTN_VARLEN_ERR_SCRATCH_TOO_SMALL:
      return "the problem needs more workspace than the static scratch of the allocation-free call holds";
    default: return "unknown error code";
  }
}

int attn_varlen_version(void) { return (kVersionMajor << 16) | kVersionMinor; }

int64_t attn_varlen_schedule_host(const int32_t* cu_seqlens_q_host, int32_t num_seqs, int32_t block_m,
                                  int32_t* seq_out, int32_t* block_out, int64_t capacity) {
  if (!cu_seqlens_q_host || (capacity > 0 && (!seq_out || !block_out))) return ATTN_VARLEN_ERR_NULL_POINTER;
  if (num_seqs < 1 || block_m < 1) return ATTN_VARLEN_ERR_BAD_SEQLEN;
  for (int b = 0; b < num_seqs; ++b)
    if (cu_seqlens_q_host[b + 1] < cu_seqlens_q_host[b]) return ATTN_VARLEN_ERR_BAD_SEQLEN;
  return av::rank_enumerate_host(cu_seqlens_q_host, num_seqs, block_m, seq_out, block_out, capacity);
}

int attn_varlen_schedule_device(const int32_t* cu_seqlens_q, int32_t num_seqs, int32_t max_seqlen_q,
                                int32_t block_m, int32_t* seq_out, int32_t* block_out, int32_t count,
                                void* stream) {
  if (!cu_seqlens_q || !seq_out || !block_out) return ATTN_VARLEN_ERR_NULL_POINTER;
  if (num_seqs < 1 || block_m < 1 || max_seqlen_q < 0 || count < 0) return ATTN_VARLEN_ERR_BAD_SEQLEN;
  if (count == 0) return ATTN_VARLEN_OK;
  return av::launch_schedule_probe(cu_seqlens_q, num_seqs, max_seqlen_q, block_m, seq_out, block_out, count,
                                   stream) == hipSuccess
             ? ATTN_VARLEN_OK
             : ATTN_VARLEN_ERR_HIP;
}

int attn_varlen_tile_plan_host(int32_t kind, int32_t head_dim, int32_t seqlen_q, int32_t seqlen_k, int32_t causal,
                               int32_t window_left, int32_t window_right, int32_t block, int32_t* plan) {
  if (!plan) return ATTN_VARLEN_ERR_NULL_POINTER;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return ATTN_VARLEN_ERR_BAD_HEAD_DIM;
  if (causal != 0 && causal != 1) return ATTN_VARLEN_ERR_BAD_FLAG;
  if (seqlen_q < 0 || seqlen_k < 0) return ATTN_VARLEN_ERR_BAD_SEQLEN;
  const int Lq = seqlen_q, Lk = seqlen_k;
  // the window as the launchers see it for a one-sequence batch (make_fwd_args,
  // band_of): sides wider than the sequence are unbounded; causal caps the right
  const int wl = (window_left < 0 || window_left >= Lk) ? -1 : window_left;
  const int wr0 = (window_right < 0 || window_right >= Lq) ? -1 : window_right;
  const int wr = causal ? 0 : wr0;
  const bool band = wl >= 0 || wr >= 0;
  for (int i = 0; i < 8; ++i) plan[i] = 0;
  const int group = kind & (ATTN_VARLEN_PLAN_GROUP2 | ATTN_VARLEN_PLAN_GROUP4);
  kind &= ~(ATTN_VARLEN_PLAN_GROUP2 | ATTN_VARLEN_PLAN_GROUP4);
  if (group == (ATTN_VARLEN_PLAN_GROUP2 | ATTN_VARLEN_PLAN_GROUP4)) return ATTN_VARLEN_ERR_BAD_FLAG;
  if (group != 0 && kind != ATTN_VARLEN_PLAN_FWD && kind != ATTN_VARLEN_PLAN_DQ) return ATTN_VARLEN_ERR_BAD_FLAG;
  if (kind == ATTN_VARLEN_PLAN_FWD || kind == ATTN_VARLEN_PLAN_DQ) {
    // the kernels' block: block_heads(r) heads of kQueryBlock / block_heads(r) rows
    const int heads = group == ATTN_VARLEN_PLAN_GROUP4 ? 4 : group == ATTN_VARLEN_PLAN_GROUP2 ? 2 : 1;
    const int bm = av::kQueryBlock / heads, bn = av::key_tile(head_dim);
    if (block < 0 || block >= av::ceil_div(Lq, bm)) return ATTN_VARLEN_ERR_BAD_SEQLEN;
    const int q0 = block * bm - av::query_lead(Lq, bm, bn);
    // the kernels' ranges: plain attention visits every key tile and masks the
    // partial last one; a band takes the tile span of the block's rows
    av::TileSpan t{0, av::ceil_div(Lk, bn), 0, Lk / bn};
    if (band) {
      const int r0 = q0 > 0 ? q0 : 0, r1 = (q0 + bm < Lq ? q0 + bm : Lq) - 1;
      // the forward's causal / right-bound path (no left bound) leaves the
      // left side open, as its launcher does
      t = av::key_tiles(r0, r1, bn, Lq, Lk, (kind == ATTN_VARLEN_PLAN_FWD && wl < 0) ? -1 : wl, wr);
    }
    int nh = 0, lo_unmasked = t.full_lo, hi_unmasked = t.full_hi;
    if (kind == ATTN_VARLEN_PLAN_FWD) {
      // the forward runs its unmasked tiles first: [0, f_hi) without a left
      // bound; with one, nh left-edge tiles, then unmasked ones up to nm
      lo_unmasked = t.lo;
      hi_unmasked = t.full_hi;
      if (wl >= 0) {
        int nm = 0;
        av::left_edge_tiles(t.lo, t.hi, t.full_lo, t.full_hi, wl, bn, nh, nm);
        lo_unmasked = t.lo + nh;
        hi_unmasked = t.lo + nm;
      }
    } else if (hi_unmasked < lo_unmasked) {
      hi_unmasked = lo_unmasked;
    }
    const int32_t v[8] = {q0, bm, bn, t.lo, t.hi, lo_unmasked, hi_unmasked, nh};
    for (int i = 0; i < 8; ++i) plan[i] = v[i];
    return ATTN_VARLEN_OK;
  }
  if (kind == ATTN_VARLEN_PLAN_DKDV) {
    const int bnk = av::kKeyBlock, bmq = av::query_step(head_dim);
    if (block < 0 || block >= av::ceil_div(Lk, bnk)) return ATTN_VARLEN_ERR_BAD_SEQLEN;
    const int n0 = block * bnk;
    av::TileSpan s{0, av::ceil_div(Lq, bmq), 0, av::ceil_div(Lq, bmq)};
    if (band) s = av::query_steps(n0, (n0 + bnk < Lk ? n0 + bnk : Lk) - 1, bmq, Lq, Lk, wl, wr);
    const int32_t v[8] = {n0, bnk, bmq, s.lo, s.hi, s.full_lo, s.full_hi, 0};
    for (int i = 0; i < 8; ++i) plan[i] = v[i];
    return ATTN_VARLEN_OK;
  }
  return ATTN_VARLEN_ERR_BAD_FLAG;
}

int attn_varlen_exp2_fma_host(const float* x, float* y, int64_t n) {
  if (n < 0) return ATTN_VARLEN_ERR_BAD_SEQLEN;
  if (n > 0 && (!x || !y)) return ATTN_VARLEN_ERR_NULL_POINTER;
  for (int64_t i = 0; i < n; ++i) y[i] = av::exp2_fma(x[i]);
  return AV_EXP2_EMU;
}

int attn_varlen_profile_enable(int enable) { return av::prof_enable(enable); }

int attn_varlen_profile_count(void) { return av::prof_count(); }

int attn_varlen_profile_get(int index, char* name, int name_capacity, float* ms) {
  const int rc = av::prof_get(index, name, name_capacity, ms);
  if (rc == -1) return ATTN_VARLEN_ERR_BAD_SEQLEN;
  if (rc != 0) return ATTN_VARLEN_ERR_HIP;
  return ATTN_VARLEN_OK;
}

}  // extern "C"
