// C ABI of the decoder-layer glue (RMSNorm, RoPE, SwiGLU, residual add) and of causal
// GQA attention.  Validation is host code and runs before any HIP call; the contracts
// are in include/lnf4.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "lnf4.h"
#include "decoder.hpp"
#include "abi_internal.hpp"

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool a16(const void* p) { return aligned(p, 16); }

int check_rows(int64_t T, int64_t H, const char* who) {
  using lnf4::fail;
  if (T < 0 || T > (int64_t)INT32_MAX / 2) return fail(LNF4_EINVAL, "%s: T=%lld out of range", who, (long long)T);
  if (H < 8 || H % 8 != 0 || H > (1 << 24))
    return fail(LNF4_ESHAPE, "%s: width %lld must be a positive multiple of 8", who, (long long)H);
  return LNF4_OK;
}

int check_attn(int64_t T, int32_t nh, int32_t nkv, int32_t D, int64_t S, const char* who) {
  using lnf4::fail;
  if (T < 0 || T > (int64_t)INT32_MAX / 2) return fail(LNF4_EINVAL, "%s: T=%lld out of range", who, (long long)T);
  if (D != 64 && D != 128) return fail(LNF4_ESHAPE, "%s: head_dim=%d (64 or 128)", who, (int)D);
  if (nh < 1 || nkv < 1 || nh > 1024 || nh % nkv != 0)
    return fail(LNF4_ESHAPE, "%s: n_heads=%d must be a positive multiple of n_kv=%d", who, (int)nh, (int)nkv);
  if (S < 64 || S % 64 != 0) return fail(LNF4_ESHAPE, "%s: seq_len=%lld must be a positive multiple of 64", who, (long long)S);
  if (T % S != 0) return fail(LNF4_ESHAPE, "%s: T=%lld is not a whole number of sequences of %lld", who, (long long)T, (long long)S);
  return LNF4_OK;
}

}  // namespace

using namespace lnf4;

extern "C" {

int lnf4_rmsnorm_fwd(const uint16_t* x, int64_t T, int64_t H, const uint16_t* g, float eps, uint16_t* y, float* rstd,
                     hipStream_t stream) {
  const char* who = "lnf4_rmsnorm_fwd";
  int rc = check_rows(T, H, who);
  if (rc) return rc;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(LNF4_EINVAL, "%s: eps must be finite and >= 0", who);
  if (T == 0) return LNF4_OK;
  if (!x || !g || !y) return fail(LNF4_EINVAL, "%s: NULL pointer", who);
  if (!a16(x) || !a16(g) || !a16(y) || (rstd && !aligned(rstd, 4))) return fail(LNF4_EALIGN, "%s: misaligned pointer", who);
  const hipError_t e = launch_rmsnorm_fwd(x, T, H, g, eps, y, rstd, stream);
  return e == hipSuccess ? LNF4_OK : hip_fail(e, "rmsnorm forward launch");
}

int lnf4_rmsnorm_bwd(const uint16_t* x, int64_t T, int64_t H, const uint16_t* g, const float* rstd, const uint16_t* dy,
                     const uint16_t* dres, uint16_t* dx, hipStream_t stream) {
  const char* who = "lnf4_rmsnorm_bwd";
  int rc = check_rows(T, H, who);
  if (rc) return rc;
  if (T == 0) return LNF4_OK;
  if (!x || !g || !rstd || !dy || !dx) return fail(LNF4_EINVAL, "%s: NULL pointer", who);
  if (!a16(x) || !a16(g) || !a16(dy) || !a16(dx) || (dres && !a16(dres)) || !aligned(rstd, 4))
    return fail(LNF4_EALIGN, "%s: misaligned pointer", who);
  const hipError_t e = launch_rmsnorm_bwd(x, T, H, g, rstd, dy, dres, dx, stream);
  return e == hipSuccess ? LNF4_OK : hip_fail(e, "rmsnorm backward launch");
}

int lnf4_rope_table(int64_t seq_len, int32_t head_dim, double base, float* table, hipStream_t stream) {
  const char* who = "lnf4_rope_table";
  if (seq_len < 1 || seq_len > (1 << 24)) return fail(LNF4_EINVAL, "%s: seq_len=%lld out of range", who, (long long)seq_len);
  if (head_dim < 16 || head_dim % 16 != 0 || head_dim > 1024) return fail(LNF4_ESHAPE, "%s: head_dim=%d (a multiple of 16)", who, (int)head_dim);
  if (!(base > 1.0) || !std::isfinite(base)) return fail(LNF4_EINVAL, "%s: base must be finite and > 1", who);
  if (!table) return fail(LNF4_EINVAL, "%s: NULL table", who);
  if (!aligned(table, 8)) return fail(LNF4_EALIGN, "%s: table not 8-byte aligned", who);
  const hipError_t e = launch_rope_table(seq_len, head_dim, base, (float2*)table, stream);
  return e == hipSuccess ? LNF4_OK : hip_fail(e, "rope table launch");
}

int lnf4_rope(uint16_t* x, int64_t T, int32_t n_heads, int32_t head_dim, int64_t seq_len, const float* table,
              int32_t inverse, hipStream_t stream) {
  const char* who = "lnf4_rope";
  if (T < 0 || T > (int64_t)INT32_MAX / 2) return fail(LNF4_EINVAL, "%s: T=%lld out of range", who, (long long)T);
  if (head_dim < 16 || head_dim % 16 != 0 || head_dim > 1024) return fail(LNF4_ESHAPE, "%s: head_dim=%d (a multiple of 16)", who, (int)head_dim);
  if (n_heads < 1 || n_heads > 1024) return fail(LNF4_EINVAL, "%s: n_heads=%d out of range", who, (int)n_heads);
  if (seq_len < 1) return fail(LNF4_EINVAL, "%s: seq_len=%lld", who, (long long)seq_len);
  if (T == 0) return LNF4_OK;
  if (!x || !table) return fail(LNF4_EINVAL, "%s: NULL pointer", who);
  if (!a16(x) || !aligned(table, 8)) return fail(LNF4_EALIGN, "%s: misaligned pointer", who);
  const hipError_t e = launch_rope(x, T, n_heads, head_dim, seq_len, (const float2*)table, inverse ? 1 : 0, stream);
  return e == hipSuccess ? LNF4_OK : hip_fail(e, "rope launch");
}

int lnf4_swiglu_fwd(const uint16_t* g, const uint16_t* u, int64_t n, uint16_t* s, hipStream_t stream) {
  const char* who = "lnf4_swiglu_fwd";
  if (n < 0 || n % 8 != 0) return fail(LNF4_ESHAPE, "%s: n=%lld must be a non-negative multiple of 8", who, (long long)n);
  if (n == 0) return LNF4_OK;
  if (!g || !u || !s) return fail(LNF4_EINVAL, "%s: NULL pointer", who);
  if (!a16(g) || !a16(u) || !a16(s)) return fail(LNF4_EALIGN, "%s: misaligned pointer", who);
  const hipError_t e = launch_swiglu_fwd(g, u, n, s, stream);
  return e == hipSuccess ? LNF4_OK : hip_fail(e, "swiglu forward launch");
}

int lnf4_swiglu_bwd(const uint16_t* g, const uint16_t* u, const uint16_t* ds, int64_t n, uint16_t* dg, uint16_t* du,
                    hipStream_t stream) {
  const char* who = "lnf4_swiglu_bwd";
  if (n < 0 || n % 8 != 0) return fail(LNF4_ESHAPE, "%s: n=%lld must be a non-negative multiple of 8", who, (long long)n);
  if (n == 0) return LNF4_OK;
  if (!g || !u || !ds || !dg || !du) return fail(LNF4_EINVAL, "%s: NULL pointer", who);
  if (!a16(g) || !a16(u) || !a16(ds) || !a16(dg) || !a16(du)) return fail(LNF4_EALIGN, "%s: misaligned pointer", who);
  const hipError_t e = launch_swiglu_bwd(g, u, ds, n, dg, du, stream);
  return e == hipSuccess ? LNF4_OK : hip_fail(e, "swiglu backward launch");
}

int lnf4_add(const uint16_t* a, const uint16_t* b, int64_t n, uint16_t* out, hipStream_t stream) {
  const char* who = "lnf4_add";
  if (n < 0 || n % 8 != 0) return fail(LNF4_ESHAPE, "%s: n=%lld must be a non-negative multiple of 8", who, (long long)n);
  if (n == 0) return LNF4_OK;
  if (!a || !b || !out) return fail(LNF4_EINVAL, "%s: NULL pointer", who);
  if (!a16(a) || !a16(b) || !a16(out)) return fail(LNF4_EALIGN, "%s: misaligned pointer", who);
  const hipError_t e = launch_add(a, b, n, out, stream);
  return e == hipSuccess ? LNF4_OK : hip_fail(e, "add launch");
}

int lnf4_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t T, int32_t n_heads, int32_t n_kv,
                  int32_t head_dim, int64_t seq_len, uint16_t* o, float* lse, hipStream_t stream) {
  const char* who = "lnf4_attn_fwd";
  int rc = check_attn(T, n_heads, n_kv, head_dim, seq_len, who);
  if (rc) return rc;
  if (T == 0) return LNF4_OK;
  if (!q || !k || !v || !o || !lse) return fail(LNF4_EINVAL, "%s: NULL pointer", who);
  if (!a16(q) || !a16(k) || !a16(v) || !a16(o) || !aligned(lse, 4)) return fail(LNF4_EALIGN, "%s: misaligned pointer", who);
  const hipError_t e = launch_attn_fwd(q, k, v, T, n_heads, n_kv, head_dim, seq_len, o, lse, stream);
  return e == hipSuccess ? LNF4_OK : hip_fail(e, "attention forward launch");
}

size_t lnf4_attn_bwd_workspace(int64_t T, int32_t n_heads, int32_t n_kv, int32_t head_dim) {
  if (T < 0 || n_heads < 1 || n_kv < 1 || n_heads % n_kv != 0 || (head_dim != 64 && head_dim != 128)) return 0;
  return attn_bwd_workspace_bytes(T, n_heads, n_kv, head_dim);
}

int lnf4_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o, const float* lse,
                  const uint16_t* dout, int64_t T, int32_t n_heads, int32_t n_kv, int32_t head_dim, int64_t seq_len,
                  uint16_t* dq, uint16_t* dk, uint16_t* dv, void* workspace, size_t ws_bytes, hipStream_t stream) {
  const char* who = "lnf4_attn_bwd";
  int rc = check_attn(T, n_heads, n_kv, head_dim, seq_len, who);
  if (rc) return rc;
  if (T == 0) return LNF4_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace)
    return fail(LNF4_EINVAL, "%s: NULL pointer", who);
  if (!a16(q) || !a16(k) || !a16(v) || !a16(o) || !a16(dout) || !a16(dq) || !a16(dk) || !a16(dv) ||
      !aligned(lse, 4) || !aligned(workspace, 256))
    return fail(LNF4_EALIGN, "%s: misaligned pointer (workspace: 256 bytes)", who);
  if (ws_bytes < attn_bwd_workspace_bytes(T, n_heads, n_kv, head_dim))
    return fail(LNF4_ESHAPE, "%s: workspace of %zu bytes, %zu needed", who, ws_bytes,
                attn_bwd_workspace_bytes(T, n_heads, n_kv, head_dim));
  const hipError_t e = launch_attn_bwd(q, k, v, o, lse, dout, T, n_heads, n_kv, head_dim, seq_len, dq, dk, dv,
                                       workspace, stream);
  return e == hipSuccess ? LNF4_OK : hip_fail(e, "attention backward launch");
}

}  // extern "C"
