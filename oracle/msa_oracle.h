/*
 * msa_oracle.h — plain, slow, single-threaded CPU oracle of the MiniMax Sparse
 * Attention (MSA) forward pass, the gradient of its main branch, and the
 * index branch's KL training signal with its gradient.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code: only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no source, header, helper,
 * table or constant with the HIP library under block_sparse_gqa_02_amd/csrc/.
 *
 * Pages this follows (titles as printed on the pages):
 *   [A] "How MiniMax M3 Was Built: Sparse Attention and Native Multimodality"
 *       (aietalks.com talk summary), sections "MSA uses a lightweight index
 *       branch before sparse attention" and "Block-level retrieval makes sparse
 *       attention easier to run on GPUs".
 *   [B] "MiniMax Researcher Olive Song: Sparse Attention Cannot Be Directly
 *       Ported Across Architectures; GPU Memory Layout Dictates Design Choices"
 *       (disconfirmai.com news write-up), paragraphs 3, 5 and 6 (counted from
 *       the first paragraph after the headline).
 *   [C] "MiniMax稀疏注意力" (disconfirmai.com topic page), summary paragraph:
 *       exact attention is computed only over the selected key/value blocks.
 *   [D] talks.tomv.uk analysis of the same talk, key_points 2 and 4.
 *
 * What the pages fix: an index branch of 4 index-query heads against one
 * index-key head scores the causal context [A §index branch, D kp2]; each KV
 * head selects its own top-k set, with no merging across heads [B ¶6, D kp4];
 * selection is over blocks of tokens, not single tokens [A §block-level, B ¶6];
 * the main GQA branch then computes exact softmax attention over the selected
 * blocks only [C summary].
 *
 * What the pages leave open and this oracle fixes (the implementation's
 * constants and readings): block size is a parameter (64 in every workload);
 * a block's score is the max over the block's tokens and over the index heads
 * attributed to the KV head (index head i -> KV head i mod Hkv) of the raw
 * index dot product (no scale, no nonlinearity: a monotone map would not change
 * the selection); the query's own block is always kept (score +inf) and counts
 * toward k; ties go to the lower block index; the block score used for the
 * decision is the exact value rounded to fp32, the precision the GPU kernels
 * decide in; query head hq reads KV head hq / (Hq/Hkv); inside the own block
 * only keys j <= pos are attended.
 *
 * Precision: every dot product, softmax and weighted sum is accumulated in
 * double from the exact bf16 input values; outputs are returned as double.
 *
 * Layouts (all host memory, row-major, bf16 given as raw uint16 bit patterns):
 *   q  [B][Sq][Hq][D]        k, v [B][Hkv][Skv][D]
 *   iq [B][Sq][Hi][Di]       ik   [B][Skv][Di]
 *   seq_lens [B] (decode only: the query of sequence b sits at seq_lens[b]-1)
 * Prefill rows: row t of sequence b sits at position q_start + t.
 */
#ifndef MSA_ORACLE_H
#define MSA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t batch, seq_q, seq_kv, q_start;
  int32_t n_q_heads, n_kv_heads, head_dim;
  int32_t n_idx_heads, idx_head_dim;
  int32_t block_size, top_k;
  int32_t decode;        /* 1: positions come from seq_lens, seq_q must be 1 */
  double softmax_scale;
} oracle_problem;

enum { ORACLE_OK = 0, ORACLE_EBADARG = -1, ORACLE_ENAN = -2, ORACLE_ENOMEM = -3 };

/* Number of key blocks, ceil(seq_kv / block_size). */
int32_t oracle_num_blocks(const oracle_problem* p);

/* Position of query row (b, t); -1 on a bad argument. */
int32_t oracle_position(const oracle_problem* p, const int32_t* seq_lens, int32_t b, int32_t t);

/* Block scores of one query row, for every KV head: out[h * nblk + c].
 * c < cur: the fp32-rounded max index score; c == cur: +inf; c > cur: -inf. */
int oracle_block_scores_row(const oracle_problem* p, const uint16_t* iq, const uint16_t* ik,
                            const int32_t* seq_lens, int32_t b, int32_t t, float* out);

/* Top-k over one block-score row (length >= cur + 1): the first min(k, cur+1)
 * candidates c in [0, cur] in (score descending, c ascending) order, written
 * ascending into sel[0..k-1], the rest -1. */
int oracle_select_row(const oracle_problem* p, const float* scores, int32_t cur, int32_t* sel);

/* Exact GQA softmax attention of row (b, t) over a given selection
 * sel[h * top_k + r] (ascending block indices, -1 = none): out[hq * D + d],
 * lse[hq] = log sum exp of the scaled scores. */
int oracle_attend_row(const oracle_problem* p, const uint16_t* q, const uint16_t* k,
                      const uint16_t* v, const int32_t* seq_lens, const int32_t* sel,
                      int32_t b, int32_t t, double* out, double* lse);

/* Dense causal GQA attention of row (b, t) over every key j <= pos.
 * Written independently of oracle_attend_row. */
int oracle_dense_row(const oracle_problem* p, const uint16_t* q, const uint16_t* k,
                     const uint16_t* v, const int32_t* seq_lens, int32_t b, int32_t t,
                     double* out, double* lse);

/* The whole forward pass for a list of rows (row id = b * seq_q + t):
 * block scores -> per-KV-head selection -> attention.  Per row r:
 *   sel_out[r][Hkv][top_k], out[r][Hq][D], lse[r][Hq],
 *   scores_out[r][Hkv][nblk] (may be NULL). */
int oracle_forward_rows(const oracle_problem* p, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const uint16_t* iq, const uint16_t* ik,
                        const int32_t* seq_lens, int64_t n_rows, const int64_t* rows,
                        int32_t* sel_out, double* out, double* lse, float* scores_out);

/* The same attention as oracle_attend_row on fp64 inputs (q [B][Sq][Hq][D],
 * k, v [B][Hkv][Skv][D] as double): the forward the gradient below is the
 * derivative of, and what finite differences perturb. */
int oracle_attend_row_f64(const oracle_problem* p, const double* q, const double* k,
                          const double* v, const int32_t* seq_lens, const int32_t* sel,
                          int32_t b, int32_t t, double* out, double* lse);

/* Gradient of the main branch (the training direction the pages mention
 * without detail: [A] section "MSA uses a lightweight index branch before
 * sparse attention", kernels written for training as well as inference).
 * With out(b, t, hq) = oracle_attend_row_f64 over the selection
 * sel_all[(b * Sq + t) * Hkv * top_k + h * top_k + r] and a cotangent dout of
 * the same shape as out ([B][Sq][Hq][D], double), returns the gradients of
 * L = sum(dout * out) with respect to q, k and v:
 *   dq [B][Sq][Hq][D], dk, dv [B][Hkv][Skv][D] (all overwritten).
 * The selection is an input and receives no gradient.  Per attended token
 * a of row (b, t), head hq: p_a = softmax weight, dp_a = dout . v_a,
 * Dsum = dout . out, ds_a = p_a (dp_a - Dsum); dq += scale ds_a k_a,
 * dk_a += scale ds_a q, dv_a += p_a dout.  A row that attends nothing
 * contributes nothing. */
int oracle_attend_backward(const oracle_problem* p, const double* q, const double* k,
                           const double* v, const double* dout, const int32_t* seq_lens,
                           const int32_t* sel_all, double* dq, double* dk, double* dv);

/* Index-branch training signal ([A] section "MSA uses a lightweight index
 * branch before sparse attention": the index branch is trained with a KL
 * divergence to follow the main branch's attention).  The pages give neither
 * the direction, the distributions compared nor any scale; this oracle reads
 * them plainly.  For row (b, t) and index head i, whose KV head is
 * h = i mod Hkv, over the tokens T that KV head attends (the selected blocks
 * of sel_all, keys j <= pos; layout as for oracle_attend_backward):
 *   P_j = (1/G) sum over the G query heads hq of h of
 *         softmax_j(softmax_scale q_hq . k_j)   (the main branch, a target),
 *   Q_j = softmax_j(iq_i . ik_j)                (raw index dot products, as
 *                                                the selection uses them),
 *   loss[b][t][i] = KL(P || Q) = sum_j P_j (log P_j - log Q_j).
 * Gradients of the summed loss (double, overwritten):
 *   diq [B][Sq][Hi][Di]: sum over j in T of (Q_j - P_j) ik_j;
 *   dik [B][Skv][Di]:    sum over (t, i) attending j of (Q_j - P_j) iq_i
 *                        (zero for keys nothing attends).
 * q [B][Sq][Hq][D], k [B][Hkv][Skv][D], iq [B][Sq][Hi][Di], ik [B][Skv][Di]
 * as double.  A row with no attended token contributes nothing. */
int oracle_index_kl(const oracle_problem* p, const double* q, const double* k, const double* iq,
                    const double* ik, const int32_t* seq_lens, const int32_t* sel_all,
                    double* loss, double* diq, double* dik);

#ifdef __cplusplus
}
#endif
#endif
