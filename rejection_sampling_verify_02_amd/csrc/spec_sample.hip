// spec_sample.hip -- the batched sampler's entry points.
//
// One draw per row from the row's own distribution ("Speculative Decoding 的朴素思想",
// section "一次 sampling 怎么执行", step 1).  It is exactly the verification's bonus draw
// with no drafted positions (G = 0): the row is p_1, every position accepts vacuously,
// and the bonus token is drawn from it by inverse CDF with the row's uniform.  So the
// entry points call the verification's own C entry point with G = 0 and no draft; the
// kernels, argument checks and row codes are the same.  accepted_len becomes the row
// status (0 on a draw) and out_tokens[b, 0] the token.

#include <hip/hip_runtime.h>

#include "spec_verify.h"

extern "C" {

sv_status spec_sample_timed(const void *logits, sv_dtype dtype, const float *u, int32_t B,
                            int32_t V, float temperature, int32_t top_k, int32_t *tokens,
                            int32_t *row_status, void *workspace, size_t workspace_bytes,
                            void *stream, void *const *events, int32_t n_events,
                            int32_t *n_launched) {
  return spec_verify_timed(logits, nullptr, dtype, nullptr, nullptr, u, B, 0, V, temperature,
                           top_k, row_status, tokens, nullptr, workspace, workspace_bytes, stream,
                           events, n_events, n_launched);
}

sv_status spec_sample(const void *logits, sv_dtype dtype, const float *u, int32_t B, int32_t V,
                      float temperature, int32_t top_k, int32_t *tokens, int32_t *row_status,
                      void *workspace, size_t workspace_bytes, void *stream) {
  return spec_verify(logits, nullptr, dtype, nullptr, nullptr, u, B, 0, V, temperature, top_k,
                     row_status, tokens, nullptr, workspace, workspace_bytes, stream);
}

}  // extern "C"
