/*
 * msa.h — C ABI of libmsa.so: the forward hot path of MiniMax Sparse Attention
 * (MSA) on AMD Instinct MI355X (gfx950).
 *
 * The method, as the pages describe it:
 *   - a lightweight index branch, 4 index-query heads against a single
 *     index-key head, scores the causal context (talk summary "How MiniMax M3
 *     Was Built: Sparse Attention and Native Multimodality", section "MSA uses
 *     a lightweight index branch before sparse attention");
 *   - every KV head picks its own top-k set, the index outputs are not merged
 *     across heads, and the unit of selection is a block of tokens, not a token
 *     (same page, section "Block-level retrieval makes sparse attention easier
 *     to run on GPUs"; news write-up "MiniMax Researcher Olive Song: Sparse
 *     Attention Cannot Be Directly Ported Across Architectures; GPU Memory
 *     Layout Dictates Design Choices", paragraph 6, paragraphs counted from the
 *     first one after the headline);
 *   - the main GQA branch computes exact softmax attention over the selected
 *     blocks only (topic page "MiniMax稀疏注意力", summary paragraph).
 * Constants the pages leave open are fixed here: block size 64; a block's
 * score is the max of the raw index dot products over the block's tokens and
 * over the index heads attributed to the KV head (index head i -> KV head
 * i mod n_kv_heads); the query's own block is always kept and counts toward k;
 * ties go to the lower block index; query head hq reads KV head
 * hq / (n_q_heads / n_kv_heads); inside the own block only keys j <= pos are
 * attended.
 *
 * Token-level selection (block_size 1), the alternative the pages weigh
 * blocks against (news write-up, paragraph 6: fewer candidates make top-k
 * cheaper; talk summary, section "Block-level retrieval makes sparse attention
 * easier to run on GPUs": blocks keep reads contiguous), is accepted by
 * msa_index_block_scores, msa_topk_blocks and msa_sparse_attn_prefill at
 * prefill positions, with the same definitions read at one token per block:
 * nblk = Skv, block_scores holds one score per token (own token +inf), sel
 * lists tokens.  Every other entry point rejects it (MSA_ERR_UNSUPPORTED).
 *
 * Conventions for every entry point:
 *   - Tensors are device pointers (hipMalloc'd or equivalent), densely packed
 *     row-major in the layouts below, 16-byte aligned.  bf16 is IEEE
 *     bfloat16 (raw 16-bit).  The caller owns every buffer, including any
 *     workspace; the library never allocates, frees or synchronises.
 *   - Every call is asynchronous on `stream` (NULL = the null stream).
 *   - Arguments are validated on the host before anything is launched; a call
 *     that returns an error has launched nothing, except MSA_ERR_HIP, which
 *     reports a launch failure (detail in msa_last_error()).
 *   - Positions: prefill row t of every sequence sits at q_start + t and
 *     q_start + seq_q <= seq_kv.  Decode (seq_lens != NULL): seq_q == 1 and the
 *     query of sequence b sits at seq_lens[b] - 1 (the cache already holds the
 *     new token), 1 <= seq_lens[b] <= seq_kv (values are read on the device and
 *     are not validated on the host).  cur(t) = pos(t) / 64 is the own block.
 *
 * Layouts (B batch, Sq query rows, Skv = seq_kv, Hq/Hkv query/KV heads,
 * D = 128, Hi = 4 index heads, Di = 64, nblk = ceil(Skv / 64), k = top_k):
 *   q        [B][Sq][Hq][D]     bf16      out  [B][Sq][Hq][D] bf16
 *   k, v     [B][Hkv][Skv][D]   bf16      lse  [B][Hq][Sq]    fp32 (natural log)
 *   iq       [B][Sq][Hi][Di]    bf16      ik   [B][Skv][Di]   bf16 (one index-key head)
 *   block_scores [B][Hkv][Sq][nblk] fp32  sel  [B][Hkv][Sq][k] int32
 * K/V are head-major so that one (head, block) is one contiguous 16 KiB read:
 * the pages note that splitting a head dimension over several KV heads breaks
 * contiguous reads and that block retrieval restores them (talk summary,
 * section "DeepSeek's DSA did not directly fit MiniMax's grouped-query
 * architecture").
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_ABI_VERSION 6

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARGUMENT = 1,   /* NULL/misaligned pointer, inconsistent sizes */
  MSA_ERR_UNSUPPORTED = 2,        /* valid problem outside what the kernels implement */
  MSA_ERR_WORKSPACE_TOO_SMALL = 3,
  MSA_ERR_HIP = 4                 /* a HIP launch failed; see msa_last_error() */
} msa_status;

typedef struct {
  int32_t batch;          /* B >= 1 */
  int32_t seq_q;          /* Sq >= 1 query rows per sequence (1 for decode) */
  int32_t seq_kv;         /* Skv >= 1: token capacity of k, v, ik per sequence */
  int32_t q_start;        /* prefill: position of row 0; ignored in decode */
  int32_t n_q_heads;      /* Hq */
  int32_t n_kv_heads;     /* Hkv in {1, 2, 4}; Hq / Hkv <= 16 (4 and 8 take the tiled kernels) */
  int32_t head_dim;       /* must be 128 */
  int32_t n_idx_heads;    /* must be 4 (the pages' index branch), multiple of Hkv */
  int32_t idx_head_dim;   /* must be 64 */
  int32_t block_size;     /* 64; or 1 = token-level selection (see below) */
  int32_t top_k;          /* 1..256 blocks per KV head per query (own block included);
                             1..65536 tokens at block_size 1 */
  float softmax_scale;    /* scale of q.k in the main branch, e.g. 1/sqrt(128); must be
                             finite and > 0 (<= 0: MSA_ERR_UNSUPPORTED) */
} msa_problem;

/* Arrival-counter region.  Launches whose work-groups hand data to each other
 * (the decode forms of msa_index_topk_fused and msa_index_topk_fused_paged,
 * where the last work-group of a sequence to finish selects its blocks) count
 * arrivals in int32 counters in the first MSA_COUNTER_REGION_BYTES of their
 * workspace.
 * That region must be zero before the first call on a workspace (e.g. a
 * zero-filled allocation); every call puts the counters it used back to zero,
 * so a workspace stays valid for every later call of any shape it is large
 * enough for.  Calls that share a workspace must not run concurrently. */
#define MSA_COUNTER_REGION_BYTES (1u << 20)

/* Operation ids for msa_workspace_bytes. */
typedef enum {
  MSA_OP_INDEX_BLOCK_SCORES = 0,
  MSA_OP_TOPK_BLOCKS = 1,
  MSA_OP_INDEX_TOPK_FUSED = 2,
  MSA_OP_SPARSE_ATTN_PREFILL = 3,
  MSA_OP_SPARSE_ATTN_DECODE = 4,
  MSA_OP_DENSE_ATTN_PREFILL = 5,
  MSA_OP_DENSE_ATTN_DECODE = 6,
  MSA_OP_SPARSE_ATTN_PREFILL_BACKWARD = 7,
  MSA_OP_INDEX_TOPK_FUSED_DECODE = 8,  /* msa_index_topk_fused / _paged with seq_lens */
  MSA_OP_INDEX_KL_BACKWARD = 9
} msa_op;

/* Index branch: block scores.  For every sequence b, KV head h, row t and
 * block c: c < cur(t): max over index heads i with i mod Hkv == h and tokens
 * j in [64c, 64c+63] of sum_d iq[b][t][i][d] * ik[b][j][d] (bf16 products,
 * fp32 accumulation); c == cur(t): +inf; entries c > cur(t) are not written.
 * seq_lens == NULL selects prefill positions, else decode positions.  iq and
 * ik must be finite: NaN or infinite inputs give unspecified block scores.
 * Source: talk summary, section "MSA uses a lightweight index branch before
 * sparse attention" (4 index-query heads, 1 index-key head, highest-scoring
 * positions are kept); block granularity: section "Block-level retrieval
 * makes sparse attention easier to run on GPUs". */
msa_status msa_index_block_scores(const msa_problem* p, const void* iq, const void* ik,
                                  const int32_t* seq_lens, float* block_scores,
                                  hipStream_t stream);

/* Per-KV-head causal top-k over block scores.  For every (b, h, t): the first
 * min(k, cur+1) blocks c in [0, cur] in order of (score descending, c
 * ascending), with the own block cur treated as +inf whatever block_scores
 * holds there; written ascending into sel[b][h][t][0..], the rest -1.  Scores
 * compare as reals (-0 == +0); NaN scores give an unspecified selection.
 * Source: news write-up, paragraph 6 (each KV head selects independently, no
 * aggregation; fewer candidates make top-k and merging cheaper). */
msa_status msa_topk_blocks(const msa_problem* p, const float* block_scores,
                           const int32_t* seq_lens, int32_t* sel, hipStream_t stream);

/* Index scoring and top-k in one pass: the same sel as msa_index_block_scores
 * followed by msa_topk_blocks.
 * Prefill positions (seq_lens == NULL): block scores stream through a running
 * top-k and are never written to memory (needed at 1M-token contexts, where
 * they would take gigabytes).  workspace: msa_workspace_bytes(p,
 * MSA_OP_INDEX_TOPK_FUSED) bytes, any content; it holds per-split candidate
 * lists.
 * Decode positions (seq_lens != NULL): one launch scores every sequence's
 * index-K cache and selects its blocks (the work-groups of a sequence count
 * themselves in after writing its block scores; the last one selects).
 * workspace: msa_workspace_bytes(p, MSA_OP_INDEX_TOPK_FUSED_DECODE) bytes: the
 * arrival-counter region (see below), then the block scores [B][Hkv][nblk]
 * fp32.  Sequences times (1 + ceil(nblk / 512)) must not exceed the 262144
 * counters of the region (MSA_ERR_UNSUPPORTED).
 * iq and ik must be finite, as for msa_index_block_scores.
 * Source: as msa_index_block_scores and msa_topk_blocks; the 1M-token window
 * is named in the talk summary, section "MiniMax M3 combines agentic coding,
 * long context, and native multimodality"; decode speed-ups in the news
 * write-up, paragraph 7. */
msa_status msa_index_topk_fused(const msa_problem* p, const void* iq, const void* ik,
                                const int32_t* seq_lens, int32_t* sel, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* Main branch, prefill: exact GQA softmax attention of every row over the
 * tokens of the blocks its KV head selected.  For query head hq (KV head
 * h = hq / (Hq/Hkv)): T = { j : j/64 in sel[b][h][t][:], j <= pos(t) },
 * out = softmax(softmax_scale * q.k_j over T) . v_j, lse = log sum exp.
 * sel entries must be -1 or in [0, cur(t)] (others give unspecified results,
 * never out-of-range reads); a row whose list is all -1 gets out = 0,
 * lse = -inf.  lse may be NULL.  bf16 operands, fp32 accumulation and softmax.
 * At block_size 1 a row's list holds distinct tokens and is read up to its
 * first entry outside [0, pos(t)] (the -1 padding of msa_topk_blocks).
 * workspace: msa_workspace_bytes(p, MSA_OP_SPARSE_ATTN_PREFILL) bytes, any
 * content (may be NULL when that is 0).  For n_q_heads / n_kv_heads of 4 or 8
 * at block_size 64 it receives a transposed copy of V's context blocks,
 * B * n_kv_heads * ceil((q_start + seq_q) / 64) * 16 KiB, which the kernel
 * streams instead of V, followed by a 256-byte status block.
 * Failure mode: the work-groups of that kernel share K/V blocks through an LDS
 * ring with bounded waits; a wait that exceeds its bound (never expected; it
 * exists so that a fault elsewhere cannot hang the GPU) ends the call early
 * and normally: the affected rows get NaN outputs and LSE, and the int32 word
 * at msa_sparse_attn_prefill_status_offset() in the workspace reads 1 once the
 * call has completed on the stream (0 after a complete call; the call clears
 * it before its sweep).  The return value is MSA_OK either way, since nothing
 * is known on the host when the call returns.
 * Source: topic page "MiniMax稀疏注意力", summary paragraph (exact attention
 * only over the selected blocks). */
msa_status msa_sparse_attn_prefill(const msa_problem* p, const void* q, const void* k,
                                   const void* v, const int32_t* sel, void* out, float* lse,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Main branch, decode: as msa_sparse_attn_prefill for the single query of
 * each sequence at seq_lens[b] - 1, with the selected blocks split over
 * several work-groups whose partial softmax states are merged by
 * log-sum-exp.  workspace: msa_workspace_bytes(p, MSA_OP_SPARSE_ATTN_DECODE)
 * bytes, any content (it receives the split partials).
 * Source: as msa_sparse_attn_prefill; decode speed-ups over full attention are
 * reported in the news write-up, paragraph 7. */
msa_status msa_sparse_attn_decode(const msa_problem* p, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* seq_lens,
                                  const int32_t* sel, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* msa_sparse_attn_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and results, with the split partials in a
 * scratch array of 16 MiB that the library itself holds on every GPU it runs
 * on until the process ends, instead of a caller's workspace.  The call
 * allocates nothing.  The scratch is that of the device current on the calling
 * thread (stream must belong to it); its address is looked up on the first
 * call on a device.  A problem that needs more than 16 MiB of partials
 * (msa_workspace_bytes(p, MSA_OP_SPARSE_ATTN_DECODE) > 16 MiB; 32 sequences of
 * 4 KV heads at top_k 64 need 4.3 MB) returns MSA_ERR_WORKSPACE_TOO_SMALL
 * and launches nothing.  Every call on a GPU shares that GPU's one scratch:
 * calls that overlap on one GPU (other streams, other threads) race and must
 * be serialised by the caller.  Each call overwrites what it uses and needs
 * no clearing. */
msa_status msa_sparse_attn_decode_static(const msa_problem* p, const void* q, const void* k_cache,
                                         const void* v_cache, const int32_t* seq_lens,
                                         const int32_t* sel, void* out, float* lse,
                                         hipStream_t stream);

/* Dense causal GQA attention over every key j <= pos(t): the full-attention
 * baseline that the pages quote every speed-up against (news write-up,
 * paragraph 7: about 9x prefill and 15x decode; topic page "MiniMax稀疏注意力",
 * summary paragraph: 14.2x prefill and 7.6x decode over full attention on
 * H800).  top_k is ignored; the workspace is unused (may be NULL). */
msa_status msa_dense_attn_prefill(const msa_problem* p, const void* q, const void* k,
                                  const void* v, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* Dense decode: every key j < seq_lens[b], split over work-groups and merged by
 * log-sum-exp; the full-attention baseline of the decode speed-ups (news
 * write-up, paragraph 7; topic page "MiniMax稀疏注意力", summary paragraph).
 * workspace: msa_workspace_bytes(p, MSA_OP_DENSE_ATTN_DECODE), any content. */
msa_status msa_dense_attn_decode(const msa_problem* p, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* seq_lens, void* out,
                                 float* lse, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Paged decode caches.  The index-K, K and V caches of the decode functions
 * above can instead live in page pools, one page per 64-token block:
 *   ik_pages [num_pages][64][64] bf16,  k_pages / v_pages [num_pages][Hkv][64][128]
 *   bf16 (one page and KV head is a contiguous 16 KiB run, as in the
 *   contiguous cache), page_table [batch][ceil(seq_kv / 64)] int32 (device):
 *   block c of sequence b is page page_table[b][c].
 * p->seq_kv is the capacity per sequence (it sizes page_table rows and
 * block_scores rows); only entries for blocks c <= (seq_lens[b] - 1) / 64 are
 * read.  A page id outside [0, num_pages) is never read: its block scores
 * -inf in msa_index_block_scores_paged and is skipped by
 * msa_sparse_attn_decode_paged (a caller error with unspecified selection or
 * output, not a fault).  Results are those of the contiguous functions on
 * the gathered caches, bit for bit.
 * Source: the operations are those of msa_index_block_scores and
 * msa_sparse_attn_decode; the pages fix no cache layout beyond block-contiguous
 * reads (talk summary, section "Block-level retrieval makes sparse attention
 * easier to run on GPUs"), which one page per block keeps. */
msa_status msa_index_block_scores_paged(const msa_problem* p, const void* iq,
                                        const void* ik_pages, const int32_t* page_table,
                                        int32_t num_pages, const int32_t* seq_lens,
                                        float* block_scores, hipStream_t stream);

/* The decode form of msa_index_topk_fused on a paged index-K cache (same
 * workspace and counter rules; pages as for msa_index_block_scores_paged). */
msa_status msa_index_topk_fused_paged(const msa_problem* p, const void* iq, const void* ik_pages,
                                      const int32_t* page_table, int32_t num_pages,
                                      const int32_t* seq_lens, int32_t* sel, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* workspace: as msa_sparse_attn_decode. */
msa_status msa_sparse_attn_decode_paged(const msa_problem* p, const void* q,
                                        const void* k_pages, const void* v_pages,
                                        const int32_t* page_table, int32_t num_pages,
                                        const int32_t* seq_lens, const int32_t* sel, void* out,
                                        float* lse, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/* Gradient of the main branch, prefill (the pages mention kernels written for
 * training as well as inference without detail: talk summary "How MiniMax M3
 * Was Built", section "MSA uses a lightweight index branch before sparse
 * attention").  For the attention msa_sparse_attn_prefill computes over the
 * selection sel, returns the gradients of sum(dout * out) with respect to q,
 * k and v; the selection gets none.  Per attended token j of row t, query
 * head hq: p_j = exp(softmax_scale q.k_j - lse), Dsum = dout . out,
 * ds_j = p_j (dout . v_j - Dsum); dq = softmax_scale sum_j ds_j k_j,
 * dk_j += softmax_scale ds_j q, dv_j += p_j dout, summed over every row and
 * query head that attends j.
 * Inputs (device): q, dout [B][Sq][Hq][128] bf16; k, v [B][Hkv][Skv][128]
 * bf16; sel [B][Hkv][Sq][top_k] as for msa_sparse_attn_prefill, with each
 * block at most once per list; out (bf16, [B][Sq][Hq][128]) and lse (fp32,
 * [B][Hq][Sq], natural log) as msa_sparse_attn_prefill returned them for
 * these inputs.  Outputs (device, fp32, fully overwritten): dq
 * [B][Sq][Hq][128]; dk, dv [B][Hkv][Skv][128] (zero for keys no row attends).
 * Hq / Hkv must divide 64; seq_kv at most 1310720 (the inverse selection's
 * block bitmap lives in LDS).  workspace: msa_workspace_bytes(p,
 * MSA_OP_SPARSE_ATTN_PREFILL_BACKWARD) bytes, any contents.  bf16 products
 * (P and dS rounded to bf16, as P is in the forward), fp32 accumulation;
 * deterministic (no floating-point atomics).  For group sizes 4 and 8 the dq
 * pass shares blocks between rows through an LDS ring with bounded waits (as
 * msa_sparse_attn_prefill does): should a wait give up (in practice only
 * under msa_set_wait_limit), the rows of the affected tiles get NaN dq and
 * the call still returns MSA_OK. */
msa_status msa_sparse_attn_prefill_backward(const msa_problem* p, const void* q, const void* k,
                                            const void* v, const int32_t* sel, const void* out,
                                            const float* lse, const void* dout, float* dq,
                                            float* dk, float* dv, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream);

/* Index-branch training signal and its gradient, prefill (talk summary "How
 * MiniMax M3 Was Built", section "MSA uses a lightweight index branch before
 * sparse attention": the index branch is trained with a KL divergence to
 * follow the main branch's attention; the pages give no formula, and this is
 * the plain reading).  For row t and index head i, with KV head h = i mod Hkv,
 * over the tokens T that h attends in sel (its selected blocks, keys j <= pos):
 *   P_j = mean over the G query heads hq of h of exp(softmax_scale q_hq.k_j
 *         - lse[hq][t])   (the main branch's weights; a target, no gradient),
 *   Q_j = softmax over T of s_j = iq_i . ik_j   (raw index dot products),
 *   loss[b][t][i] = KL(P || Q) = sum_j P_j (log P_j - log Q_j),
 *   diq[b][t][i][:] = sum_j (Q_j - P_j) ik_j,
 *   dik[b][j][:] = sum over (t, i) attending j of (Q_j - P_j) iq_i
 * (the gradients of the summed loss; zero for keys nothing attends; a row
 * that attends nothing gets loss 0 and diq 0).
 * Inputs (device): q [B][Sq][Hq][128], k [B][Hkv][Skv][128], iq [B][Sq][4][64],
 * ik [B][Skv][64] bf16; sel [B][Hkv][Sq][top_k] as for msa_sparse_attn_prefill,
 * each block at most once per list; lse (fp32, [B][Hq][Sq], natural log) as
 * msa_sparse_attn_prefill returned it for this selection.  Outputs (device,
 * fp32, fully overwritten): loss [B][Sq][4], diq [B][Sq][4][64], dik
 * [B][Skv][64].  Hq / Hkv must be 4, 8 or 16; seq_kv at most 1310720.  workspace: msa_workspace_bytes(p,
 * MSA_OP_INDEX_KL_BACKWARD) bytes, any contents.  bf16 products (P, the index
 * softmax numerators and Q - P rounded to bf16), fp32 accumulation and
 * softmax statistics; deterministic (no floating-point atomics). */
msa_status msa_index_kl_backward(const msa_problem* p, const void* q, const void* k,
                                 const void* iq, const void* ik, const int32_t* sel,
                                 const float* lse, float* loss, float* diq, float* dik,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Byte offset, inside the workspace of msa_sparse_attn_prefill for problem p,
 * of the int32 status word described there (0: complete; 1: a bounded wait
 * gave up).  MSA_ERR_UNSUPPORTED for shapes whose kernel has no bounded wait
 * (group sizes other than 4 and 8, block_size 1).  Host only. */
msa_status msa_sparse_attn_prefill_status_offset(const msa_problem* p, size_t* offset);

/* Testing only: the number of polls of a ring tag after which a wave of the
 * sparse prefill (and of its gradient's dq pass) gives up (process-wide; <= 0
 * restores the default, 2^22).  A tiny bound forces the failure paths above
 * with every kernel still exiting normally. */
void msa_set_wait_limit(int32_t polls);

/* Workspace bytes an operation needs for problem p (0 if none).  Host only. */
msa_status msa_workspace_bytes(const msa_problem* p, msa_op op, size_t* bytes);

/* Static description of a status code. */
const char* msa_status_string(msa_status s);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* msa_last_error(void);

/* MSA_ABI_VERSION of the loaded library. */
int msa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
