// Launchers of the decoder-layer glue kernels (decoder.hip) and of causal GQA attention
// (attention.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace lnf4 {

hipError_t launch_rmsnorm_fwd(const uint16_t* x, int64_t T, int64_t H, const uint16_t* g, float eps, uint16_t* y,
                              float* rstd, hipStream_t s);
hipError_t launch_rmsnorm_bwd(const uint16_t* x, int64_t T, int64_t H, const uint16_t* g, const float* rstd,
                              const uint16_t* dy, const uint16_t* dres, uint16_t* dx, hipStream_t s);
hipError_t launch_rope_table(int64_t seq_len, int D, double base, float2* table, hipStream_t s);
hipError_t launch_rope(uint16_t* x, int64_t T, int n_heads, int D, int64_t seq_len, const float2* table, int inverse,
                       hipStream_t s);
hipError_t launch_swiglu_fwd(const uint16_t* g, const uint16_t* u, int64_t n, uint16_t* out, hipStream_t s);
hipError_t launch_swiglu_bwd(const uint16_t* g, const uint16_t* u, const uint16_t* ds, int64_t n, uint16_t* dg,
                             uint16_t* du, hipStream_t s);
hipError_t launch_add(const uint16_t* a, const uint16_t* b, int64_t n, uint16_t* out, hipStream_t s);
hipError_t launch_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t T, int nh, int nkv, int D,
                           int64_t S, uint16_t* o, float* lse, hipStream_t s);
size_t attn_bwd_workspace_bytes(int64_t T, int nh, int nkv, int D);
hipError_t launch_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                           const float* lse, const uint16_t* dO, int64_t T, int nh, int nkv, int D, int64_t S,
                           uint16_t* dq, uint16_t* dk, uint16_t* dv, void* workspace, hipStream_t s);

}  // namespace lnf4
