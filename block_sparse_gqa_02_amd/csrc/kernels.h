// kernels.h — host-side launchers of the gfx950 kernels.  Called by the C ABI
// (api.cpp) after it has validated every argument; each launcher only derives
// grid sizes and launches on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

// Launches that hand data over between their work-groups (the decode index
// scoring with its in-launch top-k) keep their arrival counters in the first
// kCounterBytes of their workspace, the same region for every shape: zero
// before the first call on a workspace, and every call puts the counters it
// used back to zero, so a workspace stays valid for any later call of any shape.
constexpr size_t kCounterBytes = 1 << 20;
constexpr int kMaxCounters = (int)(kCounterBytes / sizeof(int32_t));

struct Shape {
  int B, Sq, Skv, q_start;
  int Hq, Hkv, G;     // query heads, KV heads, Hq / Hkv
  int top_k;
  float scale;        // main-branch softmax scale
  int nblk;           // ceil(Skv / bs)
  int bs;             // tokens per selection block: 64, or 1 (token-level selection)
};

// Paged caches (decode): block c of sequence b lives in page table[b * nblk + c]
// of pools of num_pages pages; ids outside [0, num_pages) are never read.
struct Paging {
  const int32_t* table;
  int num_pages;
};

// Index branch: block scores [B][Hkv][Sq][nblk] (decode when seq_lens != NULL).
// pg (decode only): ik is a pool of [num_pages][64][64] pages.
hipError_t launch_index_block_scores(const Shape& s, const void* iq, const void* ik,
                                     const int32_t* seq_lens, float* scores, hipStream_t st,
                                     const Paging* pg = nullptr);

// Decode index scoring and top-k in one launch: block scores into the workspace,
// each sequence's selection by its last work-group.  Workspace: the fixed
// arrival-counter region (zero before the first call on a buffer; every call
// leaves it zero), then the block scores.
size_t index_topk_decode_workspace_bytes(const Shape& s);
bool index_topk_decode_counters_fit(const Shape& s);
hipError_t launch_index_topk_decode(const Shape& s, const void* iq, const void* ik,
                                    const int32_t* seq_lens, int32_t* sel, void* ws,
                                    size_t ws_bytes, hipStream_t st, const Paging* pg = nullptr);

// Per-KV-head top-k over block scores -> sel [B][Hkv][Sq][k].
hipError_t launch_topk_blocks(const Shape& s, const float* scores, const int32_t* seq_lens,
                              int32_t* sel, hipStream_t st);

// Fused index scoring + running top-k (prefill).
size_t fused_workspace_bytes(const Shape& s);

// Main-branch gradient (prefill): dq [B][Sq][Hq][128], dk, dv [B][Hkv][Skv][128]
// in fp32 from q, k, v, dout (bf16), the selection, the forward output (bf16)
// and log-sum-exp ([B][Hq][Sq]).
size_t sparse_bwd_workspace_bytes(const Shape& s);
hipError_t launch_sparse_attn_backward(const Shape& s, const void* q, const void* k, const void* v,
                                       const int32_t* sel, const void* out, const float* lse,
                                       const void* dout, float* dq, float* dk, float* dv, void* ws,
                                       hipStream_t st);
// The rows that selected each (sequence, KV head, block), ascending, built
// from sel [B][Hkv][Sq][top_k] in ws (inverse_lists_bytes(s) bytes): list
// starts base[(b * Hkv + h) * nblk + c] (then the total) into lists.  With
// slotpos ([B][Hkv][Sq][top_k]), also the list position of every selection
// entry (-1 where the entry attends nothing).
size_t inverse_lists_bytes(const Shape& s);
hipError_t launch_inverse_lists(const Shape& s, const int32_t* sel, void* ws,
                                const int32_t** base, const int32_t** lists, hipStream_t st,
                                int32_t* slotpos = nullptr);

// Index-branch KL gradient (prefill): loss [B][Sq][4], diq [B][Sq][4][64],
// dik [B][Skv][64] in fp32 from q, k, iq, ik (bf16), the selection and the
// forward's log-sum-exp ([B][Hq][Sq]).
bool index_kl_supported(const Shape& s);
size_t index_kl_workspace_bytes(const Shape& s);
hipError_t launch_index_kl_backward(const Shape& s, const void* q, const void* k, const void* iq,
                                    const void* ik, const int32_t* sel, const float* lse,
                                    float* loss, float* diq, float* dik, void* ws,
                                    hipStream_t st);
hipError_t launch_index_topk_fused(const Shape& s, const void* iq, const void* ik, int32_t* sel,
                                   void* ws, hipStream_t st);

// Sparse attention.  ws: sparse_prefill_workspace_bytes(s) bytes (the
// tile-union kernel's transposed V tiles; unused by the row-wise kernel).
size_t sparse_prefill_workspace_bytes(const Shape& s);
// Byte offset of the int32 status word in that workspace (tiled schedules).
size_t sparse_prefill_status_offset(const Shape& s);
hipError_t launch_sparse_attn_prefill(const Shape& s, const void* q, const void* k,
                                      const void* v, const int32_t* sel, void* out, float* lse,
                                      void* ws, hipStream_t st);
// Tile-union schedule of the sparse prefill (used for G = 4 and 8).
bool union_prefill_supported(const Shape& s);
size_t union_prefill_workspace_bytes(const Shape& s);
// Byte offset of the int32 failure word in the tile-union workspace.
size_t union_prefill_status_offset(const Shape& s);
// Polls of a ring tag before a wave gives up (<= 0 restores the default); the
// bound of every ring kernel (tile-union prefill and its dQ).
void set_union_spin_limit(int spins);
int union_spin_limit();
hipError_t launch_union_prefill(const Shape& s, const void* q, const void* k, const void* v,
                                const int32_t* sel, void* out, float* lse, void* ws,
                                hipStream_t st);
// The transposed V tiles of the context (start of ws), and the status word
// after them cleared; shared by both tiled schedules.
hipError_t launch_vt_tiles(const Shape& s, const void* v, void* ws, hipStream_t st);
// KV-block-stationary schedule of the sparse prefill (G = 4 and 8), used when a
// tile-union tile's rows would select fewer blocks than the context holds.
// Its workspace starts with the 256-byte status word.
bool kvs_prefill_preferred(const Shape& s);
size_t kvs_prefill_workspace_bytes(const Shape& s);
hipError_t launch_kvs_prefill(const Shape& s, const void* q, const void* k, const void* v,
                              const int32_t* sel, void* out, float* lse, void* ws,
                              hipStream_t st);
// Decode workspace: the split partials (any content).
size_t decode_workspace_bytes(const Shape& s, bool dense);
// The library's static decode scratch on the current device: its size, and
// its device address (hipGetSymbolAddress on the first call per device).
size_t decode_scratch_bytes();
hipError_t decode_scratch(void** ptr);
// sel == NULL: dense; pg: k and v are pools of [num_pages][Hkv][64][128] pages.
hipError_t launch_attn_decode(const Shape& s, const void* q, const void* k, const void* v,
                              const int32_t* seq_lens, const int32_t* sel, void* out, float* lse,
                              void* ws, size_t ws_bytes, hipStream_t st,
                              const Paging* pg = nullptr);

// Token-level selection (block size 1, prefill positions): token scores
// [B][Hkv][Sq][Skv] (entries j <= pos written), per-KV-head top-k over them,
// and attention over the selected tokens.
hipError_t launch_token_scores(const Shape& s, const void* iq, const void* ik, float* scores,
                               hipStream_t st);
hipError_t launch_token_topk(const Shape& s, const float* scores, int32_t* sel, hipStream_t st);
hipError_t launch_token_attn_prefill(const Shape& s, const void* q, const void* k, const void* v,
                                     const int32_t* sel, void* out, float* lse, hipStream_t st);

// Dense causal attention (baseline): row-wise (one wave per row and KV head)
// and tiled (K/V tiles shared by a work-group of rows).
hipError_t launch_dense_attn_prefill_rowwise(const Shape& s, const void* q, const void* k,
                                             const void* v, void* out, float* lse,
                                             hipStream_t st);
hipError_t launch_dense_attn_prefill(const Shape& s, const void* q, const void* k, const void* v,
                                     void* out, float* lse, hipStream_t st);

}  // namespace msa
