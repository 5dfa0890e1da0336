// C ABI of the output side of a step: embedding gather, token cross-entropy, sequence
// sums and the sigmoid preference loss.  Validation is host code and runs before any HIP
// call (the embedding gather then asks the runtime what kind of memory its table is); the
// contracts are in include/lnf4.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "lnf4.h"
#include "head.hpp"
#include "abi_internal.hpp"

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

}  // namespace

using namespace lnf4;

extern "C" {

int lnf4_embed_gather(const uint16_t* table, int64_t vocab, int64_t hidden, const int32_t* ids, int64_t T,
                      uint16_t* out, hipStream_t stream) {
  const char* who = "lnf4_embed_gather";
  if (T < 0 || T > (int64_t)INT32_MAX / 2) return fail(LNF4_EINVAL, "%s: T=%lld out of range", who, (long long)T);
  if (vocab < 1 || vocab > (int64_t)INT32_MAX) return fail(LNF4_ESHAPE, "%s: vocab=%lld out of range", who, (long long)vocab);
  if (hidden < 8 || hidden % 8 != 0 || hidden > (1 << 24))
    return fail(LNF4_ESHAPE, "%s: hidden=%lld must be a positive multiple of 8", who, (long long)hidden);
  if (T == 0) return LNF4_OK;
  if (!table || !ids || !out) return fail(LNF4_EINVAL, "%s: NULL pointer", who);
  if (!aligned(table, 16) || !aligned(out, 16) || !aligned(ids, 4)) return fail(LNF4_EALIGN, "%s: misaligned pointer", who);
  // the table may be device memory or page-locked host memory mapped for the device (the
  // rows are then read over the host link): ask the runtime which, and take the device's
  // address of a host table, so that a pointer the device cannot read is refused here
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof attr);
  if (hipPointerGetAttributes(&attr, table) != hipSuccess) {
    (void)hipGetLastError();
    return fail(LNF4_EINVAL, "%s: table is neither device memory nor page-locked host memory", who);
  }
  const uint16_t* dtab = table;
  if (attr.type == hipMemoryTypeHost) {
    if (!attr.devicePointer) return fail(LNF4_EINVAL, "%s: the page-locked host table is not mapped for the device", who);
    dtab = (const uint16_t*)((const char*)attr.devicePointer + ((const char*)table - (const char*)attr.hostPointer));
    if (!aligned(dtab, 16)) return fail(LNF4_EALIGN, "%s: misaligned device address of the host table", who);
  }
  const hipError_t e = launch_embed_gather(dtab, vocab, hidden, ids, T, out, stream);
  return e == hipSuccess ? LNF4_OK : hip_fail(e, "embed gather launch");
}

int lnf4_cross_entropy(const uint16_t* logits, int64_t T, int64_t vocab, const int32_t* labels, float grad_scale,
                       const float* seq_scale, int64_t rows_per_scale, float* logp, uint16_t* dlogits,
                       hipStream_t stream) {
  const char* who = "lnf4_cross_entropy";
  if (T < 0 || T > (int64_t)INT32_MAX / 2) return fail(LNF4_EINVAL, "%s: T=%lld out of range", who, (long long)T);
  if (vocab < 8 || vocab % 8 != 0 || vocab > (int64_t)INT32_MAX)
    return fail(LNF4_ESHAPE, "%s: vocab=%lld must be a positive multiple of 8", who, (long long)vocab);
  if (!std::isfinite(grad_scale)) return fail(LNF4_EINVAL, "%s: grad_scale is not finite", who);
  if (seq_scale && rows_per_scale < 1)
    return fail(LNF4_EINVAL, "%s: rows_per_scale=%lld must be >= 1 with seq_scale", who, (long long)rows_per_scale);
  if (T == 0) return LNF4_OK;
  if (!logits || !labels) return fail(LNF4_EINVAL, "%s: NULL logits or labels", who);
  if (!logp && !dlogits) return fail(LNF4_EINVAL, "%s: neither logp nor dlogits requested", who);
  if (!aligned(logits, 16) || !aligned(labels, 4) || (dlogits && !aligned(dlogits, 16)) ||
      (logp && !aligned(logp, 4)) || (seq_scale && !aligned(seq_scale, 4)))
    return fail(LNF4_EALIGN, "%s: misaligned pointer", who);
  const hipError_t e = launch_cross_entropy(logits, T, vocab, labels, grad_scale, seq_scale, seq_scale ? rows_per_scale : 1,
                                            logp, dlogits, stream);
  return e == hipSuccess ? LNF4_OK : hip_fail(e, "cross-entropy launch");
}

int lnf4_sequence_sums(const float* x, int32_t n_seq, int64_t seq_len, float* sums, hipStream_t stream) {
  const char* who = "lnf4_sequence_sums";
  if (n_seq < 0) return fail(LNF4_EINVAL, "%s: n_seq=%d is negative", who, (int)n_seq);
  if (seq_len < 1 || seq_len > (int64_t)INT32_MAX) return fail(LNF4_EINVAL, "%s: seq_len=%lld out of range", who, (long long)seq_len);
  if (n_seq == 0) return LNF4_OK;
  if (!x || !sums) return fail(LNF4_EINVAL, "%s: NULL pointer", who);
  if (!aligned(x, 4) || !aligned(sums, 4)) return fail(LNF4_EALIGN, "%s: misaligned pointer", who);
  const hipError_t e = launch_sequence_sums(x, n_seq, seq_len, sums, stream);
  return e == hipSuccess ? LNF4_OK : hip_fail(e, "sequence sums launch");
}

int lnf4_dpo_loss(const float* pol_sums, const float* ref_sums, int32_t n_pairs, float beta, float* loss, float* coef,
                  hipStream_t stream) {
  const char* who = "lnf4_dpo_loss";
  if (n_pairs < 1 || n_pairs > (1 << 20)) return fail(LNF4_EINVAL, "%s: n_pairs=%d outside 1..2^20", who, (int)n_pairs);
  if (!std::isfinite(beta) || beta <= 0.0f) return fail(LNF4_EINVAL, "%s: beta must be finite and > 0", who);
  if (!pol_sums || !ref_sums || !loss || !coef) return fail(LNF4_EINVAL, "%s: NULL pointer", who);
  if (!aligned(pol_sums, 4) || !aligned(ref_sums, 4) || !aligned(loss, 4) || !aligned(coef, 4))
    return fail(LNF4_EALIGN, "%s: misaligned pointer", who);
  const hipError_t e = launch_dpo_loss(pol_sums, ref_sums, n_pairs, beta, loss, coef, stream);
  return e == hipSuccess ? LNF4_OK : hip_fail(e, "DPO loss launch");
}

}  // extern "C"
