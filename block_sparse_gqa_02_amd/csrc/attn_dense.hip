// attn_dense.hip — dense causal GQA attention (the full-attention baseline).
#include "common.h"
#include "kernels.h"

namespace msa {

hipError_t launch_dense_attn_prefill(const Shape& s, const void* q, const void* k, const void* v,
                                     void* out, float* lse, hipStream_t st) {
  return launch_dense_attn_prefill_rowwise(s, q, k, v, out, lse, st);
}

}  // namespace msa
