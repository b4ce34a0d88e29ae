// api.cpp — the C ABI of libmsa.so (include/msa.h): host-side argument
// validation, then the kernel launchers of kernels.h.  Validation touches no
// HIP API, so every error path is testable on a machine without a GPU.
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "msa.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

msa_status fail(msa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
msa_status fail(msa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

msa_status ok() {
  g_last_error.clear();
  return MSA_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// bf16 tensors and fp32 partials are moved in 16-byte vectors; int32/fp32
// per-element arrays need their natural 4-byte alignment.
#define NEED_PTR_A(p, a)                                                                 \
  do {                                                                                   \
    if ((p) == nullptr) return fail(MSA_ERR_INVALID_ARGUMENT, "%s is NULL", #p);         \
    if (!aligned((p), (a)))                                                              \
      return fail(MSA_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", #p, (int)(a));  \
  } while (0)
#define NEED_PTR(p) NEED_PTR_A(p, 16)
#define NEED_PTR4(p) NEED_PTR_A(p, 4)

enum class Mode { kPrefill, kDecode, kEither };

// Largest k of a token-level (block size 1) selection.
constexpr int kMaxTokenTopK = 65536;

// Common checks; fills the launcher's Shape.  need_k: top_k must be usable;
// tokens: the call also implements block size 1 (prefill positions only).
msa_status check_problem(const msa_problem* p, Mode mode, bool need_k, msa::Shape* s,
                         bool tokens = false) {
  if (!p) return fail(MSA_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (p->batch < 1 || p->seq_q < 1 || p->seq_kv < 1 || p->n_q_heads < 1 || p->n_kv_heads < 1 ||
      p->head_dim < 1 || p->n_idx_heads < 1 || p->idx_head_dim < 1 || p->block_size < 1)
    return fail(MSA_ERR_INVALID_ARGUMENT, "sizes must be >= 1");
  if (p->n_q_heads % p->n_kv_heads != 0)
    return fail(MSA_ERR_INVALID_ARGUMENT, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                p->n_q_heads, p->n_kv_heads);
  if (!std::isfinite(p->softmax_scale))
    return fail(MSA_ERR_INVALID_ARGUMENT, "softmax_scale is not finite");
  // the tiled kernels take the running max on unscaled scores
  if (!(p->softmax_scale > 0.f))
    return fail(MSA_ERR_UNSUPPORTED, "softmax_scale must be > 0");
  if (need_k && p->top_k < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "top_k must be >= 1");
  if (mode == Mode::kDecode && p->seq_q != 1)
    return fail(MSA_ERR_INVALID_ARGUMENT, "decode needs seq_q == 1 (got %d)", p->seq_q);
  if (mode == Mode::kPrefill &&
      (p->q_start < 0 || (int64_t)p->q_start + p->seq_q > p->seq_kv))
    return fail(MSA_ERR_INVALID_ARGUMENT, "prefill needs 0 <= q_start and q_start + seq_q <= seq_kv");
  // what the kernels implement
  if (p->head_dim != 128) return fail(MSA_ERR_UNSUPPORTED, "head_dim must be 128");
  if (p->idx_head_dim != 64) return fail(MSA_ERR_UNSUPPORTED, "idx_head_dim must be 64");
  if (p->block_size == 1) {
    if (!tokens)
      return fail(MSA_ERR_UNSUPPORTED,
                  "block_size 1 (token-level selection) is implemented by msa_index_block_scores, "
                  "msa_topk_blocks and msa_sparse_attn_prefill at prefill positions only");
    if (mode == Mode::kDecode)
      return fail(MSA_ERR_UNSUPPORTED, "block_size 1 needs prefill positions (seq_lens == NULL)");
  } else if (p->block_size != 64) {
    return fail(MSA_ERR_UNSUPPORTED, "block_size must be 64 (or 1 for token-level selection)");
  }
  if (p->n_idx_heads != 4) return fail(MSA_ERR_UNSUPPORTED, "n_idx_heads must be 4");
  if (p->n_kv_heads > 4 || 4 % p->n_kv_heads != 0)
    return fail(MSA_ERR_UNSUPPORTED, "n_kv_heads must divide the 4 index heads (1, 2 or 4)");
  const int G = p->n_q_heads / p->n_kv_heads;
  if (G > 16) return fail(MSA_ERR_UNSUPPORTED, "n_q_heads / n_kv_heads must be <= 16");
  if (need_k && p->block_size == 64 && p->top_k > 256)
    return fail(MSA_ERR_UNSUPPORTED, "top_k must be <= 256");
  if (need_k && p->block_size == 1 && p->top_k > kMaxTokenTopK)
    return fail(MSA_ERR_UNSUPPORTED, "top_k must be <= %d at block_size 1", kMaxTokenTopK);
  if (p->batch > 65535) return fail(MSA_ERR_UNSUPPORTED, "batch must be <= 65535");
  s->B = p->batch;
  s->Sq = p->seq_q;
  s->Skv = p->seq_kv;
  s->q_start = mode == Mode::kDecode ? 0 : p->q_start;
  s->Hq = p->n_q_heads;
  s->Hkv = p->n_kv_heads;
  s->G = G;
  s->top_k = p->top_k;
  s->scale = p->softmax_scale;
  s->bs = p->block_size;
  s->nblk = (p->seq_kv + p->block_size - 1) / p->block_size;
  return MSA_OK;
}

msa_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Backward-specific limits on top of check_problem.
msa_status check_backward(const msa::Shape& s) {
  if (64 % s.G != 0) return fail(MSA_ERR_UNSUPPORTED, "backward needs n_q_heads / n_kv_heads to divide 64");
  if ((size_t)s.nblk * 8 > 160 * 1024) return fail(MSA_ERR_UNSUPPORTED, "backward needs seq_kv <= 1310720");
  if ((int64_t)s.B * s.Hkv * s.Sq * s.top_k >= ((int64_t)1 << 31))
    return fail(MSA_ERR_UNSUPPORTED, "backward needs batch * n_kv_heads * seq_q * top_k < 2^31");
  return MSA_OK;
}

// Index-KL-specific limits on top of check_problem and check_backward.
msa_status check_index_kl(const msa::Shape& s) {
  msa_status st = check_backward(s);
  if (st != MSA_OK) return st;
  if (!msa::index_kl_supported(s))
    return fail(MSA_ERR_UNSUPPORTED,
                "index KL gradient needs n_q_heads / n_kv_heads in {4, 8, 16}");
  if ((size_t)3 * 1024 * 16 + (size_t)s.nblk * 4 > 160 * 1024)
    return fail(MSA_ERR_UNSUPPORTED, "index KL gradient needs seq_kv <= 1310720");
  return MSA_OK;
}

}  // namespace

extern "C" {

msa_status msa_index_block_scores(const msa_problem* p, const void* iq, const void* ik,
                                  const int32_t* seq_lens, float* block_scores,
                                  hipStream_t stream) {
  msa::Shape s;
  msa_status st = check_problem(p, seq_lens ? Mode::kDecode : Mode::kPrefill, false, &s, true);
  if (st != MSA_OK) return st;
  NEED_PTR(iq);
  NEED_PTR(ik);
  NEED_PTR4(block_scores);
  if (s.bs == 1)
    return launched(msa::launch_token_scores(s, iq, ik, block_scores, stream),
                    "msa_index_block_scores");
  return launched(msa::launch_index_block_scores(s, iq, ik, seq_lens, block_scores, stream),
                  "msa_index_block_scores");
}

msa_status msa_topk_blocks(const msa_problem* p, const float* block_scores,
                           const int32_t* seq_lens, int32_t* sel, hipStream_t stream) {
  msa::Shape s;
  msa_status st = check_problem(p, seq_lens ? Mode::kDecode : Mode::kPrefill, true, &s, true);
  if (st != MSA_OK) return st;
  NEED_PTR4(block_scores);
  NEED_PTR4(sel);
  if (s.bs == 1)
    return launched(msa::launch_token_topk(s, block_scores, sel, stream), "msa_topk_blocks");
  return launched(msa::launch_topk_blocks(s, block_scores, seq_lens, sel, stream),
                  "msa_topk_blocks");
}

// Decode form of the fused index + top-k (contiguous or paged index-K cache).
static msa_status index_topk_decode(const msa_problem* p, const void* iq, const void* ik,
                                    const msa::Paging* pg, const int32_t* seq_lens, int32_t* sel,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream,
                                    const char* name) {
  msa::Shape s;
  msa_status st = check_problem(p, Mode::kDecode, true, &s);
  if (st != MSA_OK) return st;
  NEED_PTR(iq);
  NEED_PTR(ik);
  NEED_PTR4(seq_lens);
  NEED_PTR4(sel);
  NEED_PTR(workspace);
  if (!msa::index_topk_decode_counters_fit(s))
    return fail(MSA_ERR_UNSUPPORTED, "too many sequences for the arrival counters");
  const size_t need = msa::index_topk_decode_workspace_bytes(s);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  return launched(msa::launch_index_topk_decode(s, iq, ik, seq_lens, sel, workspace,
                                                workspace_bytes, stream, pg),
                  name);
}

msa_status msa_index_topk_fused(const msa_problem* p, const void* iq, const void* ik,
                                const int32_t* seq_lens, int32_t* sel, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  msa::Shape s;
  if (seq_lens)
    return index_topk_decode(p, iq, ik, nullptr, seq_lens, sel, workspace, workspace_bytes, stream,
                             "msa_index_topk_fused");
  msa_status st = check_problem(p, Mode::kPrefill, true, &s);
  if (st != MSA_OK) return st;
  NEED_PTR(iq);
  NEED_PTR(ik);
  NEED_PTR4(sel);
  const size_t need = msa::fused_workspace_bytes(s);
  if (need > 0) {
    NEED_PTR(workspace);
    if (workspace_bytes < need)
      return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  }
  return launched(msa::launch_index_topk_fused(s, iq, ik, sel, workspace, stream),
                  "msa_index_topk_fused");
}

msa_status msa_sparse_attn_prefill(const msa_problem* p, const void* q, const void* k,
                                   const void* v, const int32_t* sel, void* out, float* lse,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  msa::Shape s;
  msa_status st = check_problem(p, Mode::kPrefill, true, &s, true);
  if (st != MSA_OK) return st;
  NEED_PTR(q);
  NEED_PTR(k);
  NEED_PTR(v);
  NEED_PTR4(sel);
  NEED_PTR(out);
  if (lse && !aligned(lse, 4)) return fail(MSA_ERR_INVALID_ARGUMENT, "lse is not 4-byte aligned");
  if (s.bs == 1)
    return launched(msa::launch_token_attn_prefill(s, q, k, v, sel, out, lse, stream),
                    "msa_sparse_attn_prefill");
  const size_t need = msa::sparse_prefill_workspace_bytes(s);
  if (need > 0) {
    NEED_PTR(workspace);
    if (workspace_bytes < need)
      return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  }
  return launched(msa::launch_sparse_attn_prefill(s, q, k, v, sel, out, lse, workspace, stream),
                  "msa_sparse_attn_prefill");
}

static msa_status decode_common(const msa_problem* p, const void* q, const void* k, const void* v,
                                const int32_t* seq_lens, const int32_t* sel, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, hipStream_t stream,
                                const char* name) {
  msa::Shape s;
  msa_status st = check_problem(p, Mode::kDecode, sel != nullptr, &s);
  if (st != MSA_OK) return st;
  NEED_PTR(q);
  NEED_PTR(k);
  NEED_PTR(v);
  NEED_PTR4(seq_lens);
  NEED_PTR(out);
  NEED_PTR(workspace);
  if (lse && !aligned(lse, 4)) return fail(MSA_ERR_INVALID_ARGUMENT, "lse is not 4-byte aligned");
  const size_t need = msa::decode_workspace_bytes(s, sel == nullptr);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  return launched(msa::launch_attn_decode(s, q, k, v, seq_lens, sel, out, lse, workspace,
                                          workspace_bytes, stream),
                  name);
}

msa_status msa_sparse_attn_decode(const msa_problem* p, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* seq_lens,
                                  const int32_t* sel, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  NEED_PTR4(sel);
  return decode_common(p, q, k_cache, v_cache, seq_lens, sel, out, lse, workspace,
                       workspace_bytes, stream, "msa_sparse_attn_decode");
}

msa_status msa_sparse_attn_decode_static(const msa_problem* p, const void* q, const void* k_cache,
                                         const void* v_cache, const int32_t* seq_lens,
                                         const int32_t* sel, void* out, float* lse,
                                         hipStream_t stream) {
  msa::Shape s;
  msa_status st = check_problem(p, Mode::kDecode, true, &s);
  if (st != MSA_OK) return st;
  NEED_PTR(q);
  NEED_PTR(k_cache);
  NEED_PTR(v_cache);
  NEED_PTR4(seq_lens);
  NEED_PTR4(sel);
  NEED_PTR(out);
  if (lse && !aligned(lse, 4)) return fail(MSA_ERR_INVALID_ARGUMENT, "lse is not 4-byte aligned");
  const size_t need = msa::decode_workspace_bytes(s, false);
  if (need > msa::decode_scratch_bytes())
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                "this problem needs %zu bytes of scratch; the library's static decode scratch "
                "holds %zu (use msa_sparse_attn_decode with a workspace)",
                need, msa::decode_scratch_bytes());
  void* scratch = nullptr;
  const hipError_t e = msa::decode_scratch(&scratch);
  if (e != hipSuccess)
    return fail(MSA_ERR_HIP, "msa_sparse_attn_decode_static: scratch address: %s",
                hipGetErrorString(e));
  return launched(msa::launch_attn_decode(s, q, k_cache, v_cache, seq_lens, sel, out, lse, scratch,
                                          msa::decode_scratch_bytes(), stream),
                  "msa_sparse_attn_decode_static");
}

msa_status msa_dense_attn_prefill(const msa_problem* p, const void* q, const void* k,
                                  const void* v, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  msa::Shape s;
  msa_status st = check_problem(p, Mode::kPrefill, false, &s);
  if (st != MSA_OK) return st;
  NEED_PTR(q);
  NEED_PTR(k);
  NEED_PTR(v);
  NEED_PTR(out);
  if (lse && !aligned(lse, 4)) return fail(MSA_ERR_INVALID_ARGUMENT, "lse is not 4-byte aligned");
  return launched(msa::launch_dense_attn_prefill(s, q, k, v, out, lse, stream),
                  "msa_dense_attn_prefill");
}

msa_status msa_dense_attn_decode(const msa_problem* p, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* seq_lens, void* out,
                                 float* lse, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  return decode_common(p, q, k_cache, v_cache, seq_lens, nullptr, out, lse, workspace,
                       workspace_bytes, stream, "msa_dense_attn_decode");
}

msa_status msa_index_block_scores_paged(const msa_problem* p, const void* iq,
                                        const void* ik_pages, const int32_t* page_table,
                                        int32_t num_pages, const int32_t* seq_lens,
                                        float* block_scores, hipStream_t stream) {
  msa::Shape s;
  msa_status st = check_problem(p, Mode::kDecode, false, &s);
  if (st != MSA_OK) return st;
  NEED_PTR(iq);
  NEED_PTR(ik_pages);
  NEED_PTR4(page_table);
  NEED_PTR4(seq_lens);
  NEED_PTR4(block_scores);
  if (num_pages < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "num_pages must be >= 1");
  const msa::Paging pg{page_table, num_pages};
  return launched(msa::launch_index_block_scores(s, iq, ik_pages, seq_lens, block_scores, stream,
                                                 &pg),
                  "msa_index_block_scores_paged");
}

msa_status msa_index_topk_fused_paged(const msa_problem* p, const void* iq, const void* ik_pages,
                                      const int32_t* page_table, int32_t num_pages,
                                      const int32_t* seq_lens, int32_t* sel, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  NEED_PTR4(page_table);
  if (num_pages < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "num_pages must be >= 1");
  const msa::Paging pg{page_table, num_pages};
  return index_topk_decode(p, iq, ik_pages, &pg, seq_lens, sel, workspace, workspace_bytes, stream,
                           "msa_index_topk_fused_paged");
}

msa_status msa_sparse_attn_decode_paged(const msa_problem* p, const void* q,
                                        const void* k_pages, const void* v_pages,
                                        const int32_t* page_table, int32_t num_pages,
                                        const int32_t* seq_lens, const int32_t* sel, void* out,
                                        float* lse, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  msa::Shape s;
  msa_status st = check_problem(p, Mode::kDecode, true, &s);
  if (st != MSA_OK) return st;
  NEED_PTR(q);
  NEED_PTR(k_pages);
  NEED_PTR(v_pages);
  NEED_PTR4(page_table);
  NEED_PTR4(seq_lens);
  NEED_PTR4(sel);
  NEED_PTR(out);
  NEED_PTR(workspace);
  if (num_pages < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "num_pages must be >= 1");
  if (lse && !aligned(lse, 4)) return fail(MSA_ERR_INVALID_ARGUMENT, "lse is not 4-byte aligned");
  const size_t need = msa::decode_workspace_bytes(s, false);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  const msa::Paging pg{page_table, num_pages};
  return launched(msa::launch_attn_decode(s, q, k_pages, v_pages, seq_lens, sel, out, lse,
                                          workspace, workspace_bytes, stream, &pg),
                  "msa_sparse_attn_decode_paged");
}

msa_status msa_sparse_attn_prefill_backward(const msa_problem* p, const void* q, const void* k,
                                            const void* v, const int32_t* sel, const void* out,
                                            const float* lse, const void* dout, float* dq,
                                            float* dk, float* dv, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream) {
  msa::Shape s;
  msa_status st = check_problem(p, Mode::kPrefill, true, &s);
  if (st != MSA_OK) return st;
  st = check_backward(s);
  if (st != MSA_OK) return st;
  NEED_PTR(q);
  NEED_PTR(k);
  NEED_PTR(v);
  NEED_PTR4(sel);
  NEED_PTR(out);
  NEED_PTR4(lse);
  NEED_PTR(dout);
  NEED_PTR(dq);
  NEED_PTR(dk);
  NEED_PTR(dv);
  NEED_PTR(workspace);
  const size_t need = msa::sparse_bwd_workspace_bytes(s);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  return launched(msa::launch_sparse_attn_backward(s, q, k, v, sel, out, lse, dout, dq, dk, dv,
                                                   workspace, stream),
                  "msa_sparse_attn_prefill_backward");
}

msa_status msa_index_kl_backward(const msa_problem* p, const void* q, const void* k,
                                 const void* iq, const void* ik, const int32_t* sel,
                                 const float* lse, float* loss, float* diq, float* dik,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  msa::Shape s;
  msa_status st = check_problem(p, Mode::kPrefill, true, &s);
  if (st != MSA_OK) return st;
  st = check_index_kl(s);
  if (st != MSA_OK) return st;
  NEED_PTR(q);
  NEED_PTR(k);
  NEED_PTR(iq);
  NEED_PTR(ik);
  NEED_PTR4(sel);
  NEED_PTR4(lse);
  NEED_PTR4(loss);
  NEED_PTR(diq);
  NEED_PTR(dik);
  NEED_PTR(workspace);
  const size_t need = msa::index_kl_workspace_bytes(s);
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes, need);
  return launched(msa::launch_index_kl_backward(s, q, k, iq, ik, sel, lse, loss, diq, dik,
                                                workspace, stream),
                  "msa_index_kl_backward");
}

msa_status msa_sparse_attn_prefill_status_offset(const msa_problem* p, size_t* offset) {
  if (!offset) return fail(MSA_ERR_INVALID_ARGUMENT, "offset is NULL");
  msa::Shape s;
  msa_status st = check_problem(p, Mode::kPrefill, true, &s, true);
  if (st != MSA_OK) return st;
  if (s.bs != 64 || !msa::union_prefill_supported(s))
    return fail(MSA_ERR_UNSUPPORTED, "this shape runs a kernel without bounded waits (no status word)");
  *offset = msa::sparse_prefill_status_offset(s);
  return ok();
}

void msa_set_wait_limit(int32_t polls) { msa::set_union_spin_limit(polls); }

msa_status msa_workspace_bytes(const msa_problem* p, msa_op op, size_t* bytes) {
  if (!bytes) return fail(MSA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  msa::Shape s;
  msa_status st;
  switch (op) {
    case MSA_OP_INDEX_BLOCK_SCORES:
    case MSA_OP_TOPK_BLOCKS:
    case MSA_OP_DENSE_ATTN_PREFILL:
      st = check_problem(p, Mode::kEither, op == MSA_OP_TOPK_BLOCKS, &s,
                         op != MSA_OP_DENSE_ATTN_PREFILL);
      if (st != MSA_OK) return st;
      *bytes = 0;
      return ok();
    case MSA_OP_SPARSE_ATTN_PREFILL:
      st = check_problem(p, Mode::kPrefill, true, &s, true);
      if (st != MSA_OK) return st;
      *bytes = s.bs == 1 ? 0 : msa::sparse_prefill_workspace_bytes(s);
      return ok();
    case MSA_OP_INDEX_TOPK_FUSED:
      st = check_problem(p, Mode::kPrefill, true, &s);
      if (st != MSA_OK) return st;
      *bytes = msa::fused_workspace_bytes(s);
      return ok();
    case MSA_OP_SPARSE_ATTN_PREFILL_BACKWARD:
      st = check_problem(p, Mode::kPrefill, true, &s);
      if (st != MSA_OK) return st;
      st = check_backward(s);
      if (st != MSA_OK) return st;
      *bytes = msa::sparse_bwd_workspace_bytes(s);
      return ok();
    case MSA_OP_INDEX_KL_BACKWARD:
      st = check_problem(p, Mode::kPrefill, true, &s);
      if (st != MSA_OK) return st;
      st = check_index_kl(s);
      if (st != MSA_OK) return st;
      *bytes = msa::index_kl_workspace_bytes(s);
      return ok();
    case MSA_OP_INDEX_TOPK_FUSED_DECODE:
      st = check_problem(p, Mode::kDecode, true, &s);
      if (st != MSA_OK) return st;
      *bytes = msa::index_topk_decode_workspace_bytes(s);
      return ok();
    case MSA_OP_SPARSE_ATTN_DECODE:
    case MSA_OP_DENSE_ATTN_DECODE:
      st = check_problem(p, Mode::kDecode, op == MSA_OP_SPARSE_ATTN_DECODE, &s);
      if (st != MSA_OK) return st;
      *bytes = msa::decode_workspace_bytes(s, op == MSA_OP_DENSE_ATTN_DECODE);
      return ok();
  }
  return fail(MSA_ERR_INVALID_ARGUMENT, "unknown op %d", (int)op);
}

const char* msa_status_string(msa_status s) {
  switch (s) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARGUMENT: return "MSA_ERR_INVALID_ARGUMENT";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_WORKSPACE_TOO_SMALL: return "MSA_ERR_WORKSPACE_TOO_SMALL";
    case MSA_ERR_HIP: return "MSA_ERR_HIP";
  }
  return "MSA_ERR_UNKNOWN";
}

const char* msa_last_error(void) { return g_last_error.c_str(); }

int msa_abi_version(void) { return MSA_ABI_VERSION; }

}  // extern "C"
