// Launchers of the output-side kernels (head.hip): embedding gather, token
// cross-entropy, sequence sums and the sigmoid preference loss.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace lnf4 {

hipError_t launch_embed_gather(const uint16_t* table, int64_t vocab, int64_t hidden, const int32_t* ids, int64_t T,
                               uint16_t* out, hipStream_t s);
hipError_t launch_cross_entropy(const uint16_t* logits, int64_t T, int64_t V, const int32_t* labels, float grad_scale,
                                const float* seq_scale, int64_t rows_per_scale, float* logp, uint16_t* dlogits,
                                hipStream_t s);
hipError_t launch_sequence_sums(const float* x, int32_t n_seq, int64_t L, float* sums, hipStream_t s);
hipError_t launch_dpo_loss(const float* pol, const float* ref, int32_t P, float beta, float* loss, float* coef,
                           hipStream_t s);

}  // namespace lnf4
