// C ABI of the lnf4 library: argument validation (pure host code, runs before any HIP
// call), error reporting, and dispatch to the kernel launchers.  Declarations and the
// contract of every entry point are in include/lnf4.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "lnf4.h"
#include "kernels.hpp"
#include "abi_internal.hpp"
#include "nf4_table.hpp"

namespace lnf4 {

static thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
  return LNF4_EHIP;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

static const float kTable[16] = LNF4_TABLE_INIT;

// --------------------------------------------------------------------------- checks
static int check_weight(const lnf4_weight* W, const char* who) {
  if (!W) return fail(LNF4_EINVAL, "%s: weight descriptor is NULL", who);
  if (W->fmt != LNF4_FMT_NF4 && W->fmt != LNF4_FMT_BF16)
    return fail(LNF4_EINVAL, "%s: unknown weight format %d", who, (int)W->fmt);
  if (!W->data) return fail(LNF4_EINVAL, "%s: weight data is NULL", who);
  if (!aligned(W->data, 16)) return fail(LNF4_EALIGN, "%s: weight data not 16-byte aligned", who);
  if (W->out_f < 1 || W->out_f > (1 << 24)) return fail(LNF4_ESHAPE, "%s: out_f=%lld out of range", who, (long long)W->out_f);
  if (W->in_f < 64 || W->in_f > (1 << 24) || W->in_f % 64 != 0)
    return fail(LNF4_ESHAPE, "%s: in_f=%lld must be a positive multiple of 64", who, (long long)W->in_f);
  // the kernels address each matrix through a buffer resource with a 31-bit byte range
  const int64_t wbytes = W->fmt == LNF4_FMT_NF4 ? W->out_f * W->in_f / 2 : W->out_f * W->in_f * 2;
  if (wbytes > (int64_t)INT32_MAX) return fail(LNF4_ESHAPE, "%s: weight of %lld bytes exceeds 2^31-1", who, (long long)wbytes);
  if (W->fmt == LNF4_FMT_NF4) {
    if (W->blocksize != 64) return fail(LNF4_ESHAPE, "%s: blocksize=%d (only 64 is supported)", who, (int)W->blocksize);
    if (!W->absmax) return fail(LNF4_EINVAL, "%s: absmax is NULL for an NF4 weight", who);
    if (!aligned(W->absmax, 4)) return fail(LNF4_EALIGN, "%s: absmax not 4-byte aligned", who);
  }
  return LNF4_OK;
}

static int check_tokens(int64_t T, const char* who) {
  if (T < 0 || T > (int64_t)INT32_MAX / 2) return fail(LNF4_EINVAL, "%s: T=%lld out of range", who, (long long)T);
  return LNF4_OK;
}

// an activation [T, features] bf16 must fit a 31-bit byte range
static int check_activation(int64_t T, int64_t features, const char* what, const char* who) {
  if (T * features * 2 > (int64_t)INT32_MAX)
    return fail(LNF4_ESHAPE, "%s: %s of %lld x %lld bf16 exceeds 2^31-1 bytes", who, what, (long long)T, (long long)features);
  return LNF4_OK;
}

// adapter state of one projection: 1 on, 0 off, <0 error
static int adapter_state(const uint16_t* A, const uint16_t* B, int32_t r, const char* who) {
  if (r < 0 || r > LNF4_MAX_RANK) return fail(LNF4_EINVAL, "%s: r=%d outside 0..%d", who, (int)r, LNF4_MAX_RANK);
  if (r == 0) return 0;
  if (!A && !B) return 0;
  if (!A || !B) return fail(LNF4_EINVAL, "%s: exactly one of A, B is NULL with r=%d", who, (int)r);
  if (!aligned(A, 16)) return fail(LNF4_EALIGN, "%s: A not 16-byte aligned", who);
  if (!aligned(B, 2)) return fail(LNF4_EALIGN, "%s: B not 2-byte aligned", who);
  return 1;
}

static size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// --------------------------------------------------------------------------- group fwd
// Workspace bytes of a grouped forward with a workspace (0: the launch is not split)
static size_t group_fwd_ws(const lnf4_proj* projs, int32_t n, int64_t T) {
  if (!projs || n < 1 || n > LNF4_MAX_GROUP || T < 1 || T > 0x7fffffff) return 0;
  int32_t of[LNF4_MAX_GROUP];
  for (int p = 0; p < n; ++p) {
    if (projs[p].W.fmt != projs[0].W.fmt || projs[p].W.in_f != projs[0].W.in_f || projs[p].W.out_f < 1 ||
        projs[p].W.out_f > 0x7fffffff || projs[0].W.in_f < 1 || projs[0].W.in_f > 0x7fffffff)
      return 0;
    of[p] = (int32_t)projs[p].W.out_f;
  }
  return fwd_split_bytes((int)T, of, n, (int)projs[0].W.in_f, projs[0].W.fmt);
}

int group_fwd_impl(const lnf4_proj* projs, int32_t n, const uint16_t* x, int64_t T, int32_t enabled,
                   void* ws, size_t ws_bytes, hipStream_t s, const char* who) {
  if (!projs) return fail(LNF4_EINVAL, "%s: projs is NULL", who);
  if (n < 1 || n > LNF4_MAX_GROUP) return fail(LNF4_EINVAL, "%s: n=%d outside 1..%d", who, (int)n, LNF4_MAX_GROUP);
  int rc = check_tokens(T, who);
  if (rc) return rc;
  if (enabled < 0 || enabled > 2)
    return fail(LNF4_EINVAL, "%s: adapters_enabled=%d (0 off, 1 on, 2 on with u already computed)", who, (int)enabled);
  int on[LNF4_MAX_GROUP];
  for (int p = 0; p < n; ++p) {
    const lnf4_proj& P = projs[p];
    if ((rc = check_weight(&P.W, who))) return rc;
    if (P.W.in_f != projs[0].W.in_f) return fail(LNF4_ESHAPE, "%s: projection %d has a different in_f", who, p);
    if (P.W.fmt != projs[0].W.fmt) return fail(LNF4_EINVAL, "%s: projection %d has a different format", who, p);
    if ((rc = check_activation(T, P.W.in_f, "x", who)) || (rc = check_activation(T, P.W.out_f, "y", who))) return rc;
    if ((rc = adapter_state(P.A, P.B, P.r, who)) < 0) return rc;
    on[p] = enabled ? rc : 0;
    if (T > 0) {
      if (!P.y) return fail(LNF4_EINVAL, "%s: y of projection %d is NULL", who, p);
      if (!aligned(P.y, 2)) return fail(LNF4_EALIGN, "%s: y not 2-byte aligned", who);
      if (on[p]) {
        if (!P.u) return fail(LNF4_EINVAL, "%s: u (fp32 [T, r] output) is required with the adapter on", who);
        if (!aligned(P.u, 4)) return fail(LNF4_EALIGN, "%s: u not 4-byte aligned", who);
      }
    }
  }
  if (T == 0) return LNF4_OK;
  if (!x) return fail(LNF4_EINVAL, "%s: x is NULL", who);
  if (!aligned(x, 16)) return fail(LNF4_EALIGN, "%s: x not 16-byte aligned", who);
  // K splits need the workspace the caller sized with lora_group_fwd_workspace
  const size_t need = ws_bytes || ws ? group_fwd_ws(projs, n, T) : 0;
  if (need > 0) {
    if (!ws) return fail(LNF4_EINVAL, "%s: workspace is NULL (%zu bytes needed)", who, need);
    if (ws_bytes < need) return fail(LNF4_ESHAPE, "%s: workspace %zu bytes < %zu needed", who, ws_bytes, need);
    if (!aligned(ws, 256)) return fail(LNF4_EALIGN, "%s: workspace not 256-byte aligned", who);
  }

  const int K = (int)projs[0].W.in_f;
  FwdArgs a;
  std::memset(&a, 0, sizeof a);
  a.part = need > 0 ? (float*)ws : nullptr;
  a.x = x;
  a.M = (int)T;
  a.K = K;
  a.n_proj = n;
  // u_p = x A_p^T for every adapted projection: they share x, so one job per run of
  // projections whose ranks sum to at most 64
  {
    RankArgs ra;
    std::memset(&ra, 0, sizeof ra);
    ra.T = (int)T;
    for (int p = 0; p < n; ++p) {
      if (!on[p] || enabled == 2) continue;  // 2: u holds x A^T from an earlier call on this x
      const lnf4_proj& P = projs[p];
      RankJob* J = ra.n_jobs > 0 ? &ra.job[ra.n_jobs - 1] : nullptr;
      if (!J || J->R + P.r > LNF4_MAX_RANK || J->n == kMaxGroup) {
        J = &ra.job[ra.n_jobs++];
        J->src = x;
        J->K = K;
        J->layout = 0;
      }
      J->W[J->n] = P.A;
      J->dst[J->n] = P.u;
      J->r[J->n] = P.r;
      J->dst_stride[J->n] = P.r;
      J->n += 1;
      J->R += P.r;
    }
    hipError_t e = launch_rank_proj(ra, s);
    if (e != hipSuccess) return hip_fail(e, "u = x A^T launch");
  }
  int tiles = 0;
  for (int p = 0; p < n; ++p) {
    const lnf4_proj& P = projs[p];
    FwdProj& q = a.p[p];
    q.w = P.W.data;
    q.absmax = P.W.absmax;
    q.y = P.y;
    q.u = on[p] ? P.u : nullptr;
    q.B = on[p] ? P.B : nullptr;
    q.out_f = (int)P.W.out_f;
    q.r = on[p] ? P.r : 0;
    q.scale = P.scale;
    q.tile_n0 = tiles;
    tiles += (int)((P.W.out_f + 255) / 256);
  }
  a.n_tiles_n = tiles;
  hipError_t e = launch_fwd(a, projs[0].W.fmt, s);
  if (e != hipSuccess) return hip_fail(e, "fused forward GEMM launch");
  return LNF4_OK;
}

// --------------------------------------------------------------------------- group bwd
// Workspace of one grouped backward call.  The adapted projections are cut into runs
// whose ranks sum to at most 64 ("chunks"); a chunk's v = dy B columns sit side by side
// in one fp32 [T][R_chunk] array, so the dA of the whole chunk is one reduction against x.
struct BwdPlan {
  int n_chunks;
  int chunk_of[LNF4_MAX_GROUP];   // chunk of projection p (-1: adapter off)
  int v_col[LNF4_MAX_GROUP];      // first column of p's v in its chunk
  int chunk_R[LNF4_MAX_GROUP];
  size_t v_off[LNF4_MAX_GROUP];   // per chunk
  size_t pa_off[LNF4_MAX_GROUP];  // per chunk: dA partials (-1: no dA asked in the chunk)
  size_t u_off[LNF4_MAX_GROUP];   // per projection: recomputed u (-1: saved or not needed)
  size_t pb_off[LNF4_MAX_GROUP];  // per projection: dB partials (-1: no dB)
  size_t dx_off;                  // split-K fp32 sums of dx (-1: the dx GEMM does not split)
  size_t total;
};

// split_ok = false: the dx GEMM is launched unsplit, so no split-K sums are planned
static void plan_bwd(const lnf4_proj* projs, int32_t n, int64_t T, const int* on, BwdPlan& pl,
                     bool split_ok = true) {
  const size_t none = (size_t)-1;
  pl.n_chunks = 0;
  for (int p = 0; p < LNF4_MAX_GROUP; ++p) {
    pl.chunk_of[p] = -1;
    pl.v_col[p] = 0;
    pl.chunk_R[p] = 0;
    pl.v_off[p] = pl.pa_off[p] = pl.u_off[p] = pl.pb_off[p] = none;
  }
  int members[LNF4_MAX_GROUP] = {0};
  for (int p = 0; p < n; ++p) {
    if (!on[p]) continue;
    const int r = projs[p].r;
    if (pl.n_chunks == 0 || pl.chunk_R[pl.n_chunks - 1] + r > LNF4_MAX_RANK) pl.n_chunks += 1;
    const int c = pl.n_chunks - 1;
    pl.chunk_of[p] = c;
    pl.v_col[p] = pl.chunk_R[c];
    pl.chunk_R[c] += r;
    members[c] += 1;
  }
  size_t off = 0;
  const int in_f = n > 0 ? (int)projs[0].W.in_f : 0;
  for (int c = 0; c < pl.n_chunks; ++c) {
    pl.v_off[c] = off;
    off += round256((size_t)T * pl.chunk_R[c] * sizeof(float));
    bool any_dA = false;
    for (int p = 0; p < n; ++p) any_dA = any_dA || (pl.chunk_of[p] == c && projs[p].dA);
    if (any_dA) {
      pl.pa_off[c] = off;
      off += round256(grad_partial_bytes((int32_t)T, in_f, pl.chunk_R[c]));
    }
  }
  for (int p = 0; p < n; ++p) {
    if (!on[p] || !projs[p].dB) continue;
    if (!projs[p].u) {
      pl.u_off[p] = off;
      off += round256((size_t)T * projs[p].r * sizeof(float));
    }
    pl.pb_off[p] = off;
    off += round256(grad_partial_bytes((int32_t)T, (int32_t)projs[p].W.out_f, projs[p].r));
  }
  // split-K sums of the dx GEMM, sized for either weight format (the workspace query of a
  // single linear does not know the format)
  int total_kb = 0;
  for (int p = 0; p < n; ++p) total_kb += (int)((projs[p].W.out_f + 63) / 64);
  size_t dxb = split_ok ? dx_split_bytes((int)T, in_f, total_kb, 0) : 0;
  const size_t dxb1 = split_ok ? dx_split_bytes((int)T, in_f, total_kb, 1) : 0;
  dxb = dxb > dxb1 ? dxb : dxb1;
  pl.dx_off = dxb ? off : none;
  off += round256(dxb);
  pl.total = off;
}

// launch a list of rank jobs in batches of kMaxJobs
// launch a list of rank jobs: one launch per layout, in batches of kMaxJobs
static hipError_t launch_rank_jobs(const RankJob* jobs, int nj, int T, hipStream_t s) {
  for (int layout = 0; layout < 2; ++layout) {
    RankArgs ra;
    std::memset(&ra, 0, sizeof ra);
    ra.T = T;
    for (int j = 0; j < nj; ++j) {
      if (jobs[j].layout != layout) continue;
      ra.job[ra.n_jobs++] = jobs[j];
      if (ra.n_jobs == kMaxJobs) {
        hipError_t e = launch_rank_proj(ra, s);
        if (e != hipSuccess) return e;
        ra.n_jobs = 0;
      }
    }
    hipError_t e = launch_rank_proj(ra, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

static hipError_t launch_grad_jobs(const GradJob* jobs, int nj, int T, int accumulate, hipStream_t s) {
  for (int j0 = 0; j0 < nj; j0 += kMaxJobs) {
    GradArgs ga;
    std::memset(&ga, 0, sizeof ga);
    ga.T = T;
    ga.accumulate = accumulate ? 1 : 0;
    ga.n_jobs = nj - j0 < kMaxJobs ? nj - j0 : kMaxJobs;
    for (int j = 0; j < ga.n_jobs; ++j) ga.job[j] = jobs[j0 + j];
    hipError_t e = launch_rank_grad(ga, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

static int bwd_adapter_flags(const lnf4_proj* projs, int32_t n, int* on, const char* who) {
  for (int p = 0; p < n; ++p) {
    int rc = adapter_state(projs[p].A, projs[p].B, projs[p].r, who);
    if (rc < 0) return rc;
    on[p] = rc;
  }
  return LNF4_OK;
}

size_t group_bwd_ws(const lnf4_proj* projs, int32_t n, int64_t T) {
  if (!projs || n < 1 || n > LNF4_MAX_GROUP || T < 0) return 0;
  int on[LNF4_MAX_GROUP];
  for (int p = 0; p < n; ++p) {
    const lnf4_proj& P = projs[p];
    on[p] = (P.r > 0 && P.r <= LNF4_MAX_RANK && P.A && P.B) ? 1 : 0;
  }
  BwdPlan pl;
  plan_bwd(projs, n, T, on, pl);
  return pl.total;
}

// ---------------------------------------------------------------- library scratch
// The workspace of lora_linear_bwd_noalloc: a fixed device array that every call on a GPU
// shares (each GPU holds its own copy, for the life of the process).  In host code the
// array's name is only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = LNF4_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static int scratch_address(void** out, const char* who) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice (library scratch)");
  if (dev < 0 || dev >= kMaxDevices) return fail(LNF4_EINVAL, "%s: device %d beyond the %d the library tracks", who, dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress (library scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LNF4_OK;
}

// lib_scratch: the workspace is the library's scratch array (ws, ws_bytes ignored); the dx
// GEMM is then never split, so the workspace holds only v, a recomputed u and the
// adapter-gradient partial sums.
int group_bwd_impl(const lnf4_proj* projs, int32_t n, const uint16_t* x, int64_t T, uint16_t* dx,
                   int32_t accumulate, void* ws, size_t ws_bytes, hipStream_t s, const char* who,
                   bool lib_scratch = false) {
  if (!projs) return fail(LNF4_EINVAL, "%s: projs is NULL", who);
  if (n < 1 || n > LNF4_MAX_GROUP) return fail(LNF4_EINVAL, "%s: n=%d outside 1..%d", who, (int)n, LNF4_MAX_GROUP);
  int rc = check_tokens(T, who);
  if (rc) return rc;
  int on[LNF4_MAX_GROUP];
  if ((rc = bwd_adapter_flags(projs, n, on, who))) return rc;
  bool need_dy = dx != nullptr, need_x = false;
  for (int p = 0; p < n; ++p) {
    const lnf4_proj& P = projs[p];
    if ((rc = check_weight(&P.W, who))) return rc;
    if (P.W.in_f != projs[0].W.in_f) return fail(LNF4_ESHAPE, "%s: projection %d has a different in_f", who, p);
    if (P.W.fmt != projs[0].W.fmt) return fail(LNF4_EINVAL, "%s: projection %d has a different format", who, p);
    if (P.W.out_f % 8 != 0) return fail(LNF4_ESHAPE, "%s: out_f=%lld must be a multiple of 8 in backward", who, (long long)P.W.out_f);
    if ((rc = check_activation(T, P.W.in_f, "x", who)) || (rc = check_activation(T, P.W.out_f, "dy", who))) return rc;
    if (on[p] && (P.dA || P.dB)) need_dy = true;
    if (on[p] && (P.dA || (P.dB && !P.u))) need_x = true;
    if (on[p] && P.dA && !aligned(P.dA, 4)) return fail(LNF4_EALIGN, "%s: dA not 4-byte aligned", who);
    if (on[p] && P.dB && !aligned(P.dB, 4)) return fail(LNF4_EALIGN, "%s: dB not 4-byte aligned", who);
    if (on[p] && P.u && !aligned(P.u, 4)) return fail(LNF4_EALIGN, "%s: u_saved not 4-byte aligned", who);
  }
  if (dx && !aligned(dx, 2)) return fail(LNF4_EALIGN, "%s: dx not 2-byte aligned", who);
  {
    int rsum = 0;
    for (int p = 0; p < n; ++p) rsum += on[p] ? projs[p].r : 0;
    if (dx && rsum > LNF4_MAX_RANK)
      return fail(LNF4_ESHAPE, "%s: the group's adapter ranks sum to %d (at most %d with dx)", who, rsum, LNF4_MAX_RANK);
  }
  if (T > 0) {
    for (int p = 0; p < n; ++p) {
      const lnf4_proj& P = projs[p];
      const bool uses_dy = dx || (on[p] && (P.dA || P.dB));
      if (uses_dy && !P.dy) return fail(LNF4_EINVAL, "%s: dy of projection %d is NULL", who, p);
      if (uses_dy && !aligned(P.dy, 16)) return fail(LNF4_EALIGN, "%s: dy not 16-byte aligned", who);
    }
    if (need_x && !x) return fail(LNF4_EINVAL, "%s: x is NULL", who);
    if (need_x && !aligned(x, 16)) return fail(LNF4_EALIGN, "%s: x not 16-byte aligned", who);
  }
  (void)need_dy;
  BwdPlan pl;
  plan_bwd(projs, n, T, on, pl, !lib_scratch);
  if (lib_scratch) {
    if (pl.total > kScratchBytes)
      return fail(LNF4_ESHAPE, "%s: these shapes need %zu bytes of scratch; the library's fixed scratch holds %zu", who,
                  pl.total, kScratchBytes);
    ws = nullptr;
    ws_bytes = kScratchBytes;
    if (pl.total > 0 && (rc = scratch_address(&ws, who))) return rc;
  }
  if (pl.total > 0) {
    if (!ws) return fail(LNF4_EINVAL, "%s: workspace is NULL (%zu bytes needed)", who, pl.total);
    if (ws_bytes < pl.total) return fail(LNF4_ESHAPE, "%s: workspace %zu bytes < %zu needed", who, ws_bytes, pl.total);
    if (!aligned(ws, 256)) return fail(LNF4_EALIGN, "%s: workspace not 256-byte aligned", who);
  }
  char* wsb = (char*)ws;
  hipError_t e;
  if (T == 0) {
    // empty batch: dx has no rows; gradients are zero (unchanged when accumulating)
    for (int p = 0; p < n; ++p) {
      const lnf4_proj& P = projs[p];
      if (!on[p] || accumulate) continue;
      if (P.dA && (e = launch_fill_zero(P.dA, (int64_t)P.r * P.W.in_f, s)) != hipSuccess) return hip_fail(e, "zero dA");
      if (P.dB && (e = launch_fill_zero(P.dB, (int64_t)P.r * P.W.out_f, s)) != hipSuccess) return hip_fail(e, "zero dB");
    }
    return LNF4_OK;
  }
  const int N = (int)projs[0].W.in_f;
  const bool any_dA = [&] {
    for (int p = 0; p < n; ++p)
      if (on[p] && projs[p].dA) return true;
    return false;
  }();
  // v = dy B per adapted projection (into its chunk's columns), and u = x A^T where dB
  // needs it and it was not saved
  const float* v[LNF4_MAX_GROUP];
  const float* u[LNF4_MAX_GROUP];
  RankJob jobs[2 * LNF4_MAX_GROUP];
  int nj = 0;
  for (int p = 0; p < n; ++p) {
    const lnf4_proj& P = projs[p];
    v[p] = u[p] = nullptr;
    if (!on[p]) continue;
    const int c = pl.chunk_of[p];
    float* vp = (float*)(wsb + pl.v_off[c]) + pl.v_col[p];
    v[p] = vp;
    if (dx || any_dA) {
      RankJob& J = jobs[nj++];
      std::memset(&J, 0, sizeof J);
      J.src = P.dy;
      J.K = (int)P.W.out_f;
      J.layout = 1;
      J.n = 1;
      J.R = P.r;
      J.W[0] = P.B;
      J.r[0] = P.r;
      J.dst[0] = vp;
      J.dst_stride[0] = pl.chunk_R[c];
    }
    if (P.dB) u[p] = P.u ? P.u : (const float*)(wsb + pl.u_off[p]);
  }
  {
    RankJob* J = nullptr;
    for (int p = 0; p < n; ++p) {
      const lnf4_proj& P = projs[p];
      if (!on[p] || !P.dB || P.u) continue;
      if (!J || J->R + P.r > LNF4_MAX_RANK) {
        J = &jobs[nj++];
        std::memset(J, 0, sizeof *J);
        J->src = x;
        J->K = N;
        J->layout = 0;
      }
      J->W[J->n] = P.A;
      J->dst[J->n] = (float*)(wsb + pl.u_off[p]);
      J->r[J->n] = P.r;
      J->dst_stride[J->n] = P.r;
      J->n += 1;
      J->R += P.r;
    }
  }
  if ((e = launch_rank_jobs(jobs, nj, (int)T, s)) != hipSuccess) return hip_fail(e, "v = dy B / u = x A^T launch");
  if (dx) {
    DxArgs a;
    std::memset(&a, 0, sizeof a);
    a.dx = dx;
    a.M = (int)T;
    a.N = N;
    a.n_proj = n;
    a.accumulate = accumulate ? 1 : 0;
    int kb = 0;
    for (int p = 0; p < n; ++p) {
      const lnf4_proj& P = projs[p];
      DxProj& q = a.p[p];
      q.w = P.W.data;
      q.absmax = P.W.absmax;
      q.dy = P.dy;
      q.v = on[p] ? v[p] : nullptr;
      q.v_stride = on[p] ? pl.chunk_R[pl.chunk_of[p]] : 0;
      q.A = on[p] ? P.A : nullptr;
      q.out_f = (int)P.W.out_f;
      q.r = on[p] ? P.r : 0;
      q.scale = P.scale;
      q.kb0 = kb;
      kb += (int)((P.W.out_f + 63) / 64);
    }
    a.total_kb = kb;
    a.part = pl.dx_off != (size_t)-1 ? (float*)(wsb + pl.dx_off) : nullptr;  // NULL: unsplit
    if ((e = launch_dx(a, projs[0].W.fmt, s)) != hipSuccess) return hip_fail(e, "fused dx GEMM launch");
  }
  // adapter gradients: dA of each chunk against x, dB of each projection against its dy
  GradJob gj[2 * LNF4_MAX_GROUP];
  int ng = 0;
  for (int c = 0; c < pl.n_chunks; ++c) {
    if (pl.pa_off[c] == (size_t)-1) continue;
    GradJob& G = gj[ng++];
    std::memset(&G, 0, sizeof G);
    G.Q = x;
    G.C = N;
    G.P = (const float*)(wsb + pl.v_off[c]);
    G.pstride = pl.chunk_R[c];
    G.R = pl.chunk_R[c];
    G.transpose = 1;
    G.part = (float*)(wsb + pl.pa_off[c]);
    for (int p = 0; p < n; ++p) {
      if (pl.chunk_of[p] != c) continue;
      G.G[G.n] = projs[p].dA;  // may be NULL: that weight's dA is skipped
      G.r[G.n] = projs[p].r;
      G.scale[G.n] = projs[p].scale;
      G.n += 1;
    }
  }
  for (int p = 0; p < n; ++p) {
    const lnf4_proj& P = projs[p];
    if (!on[p] || !P.dB) continue;
    GradJob& G = gj[ng++];
    std::memset(&G, 0, sizeof G);
    G.Q = P.dy;
    G.C = (int)P.W.out_f;
    G.P = u[p];
    G.pstride = P.r;
    G.R = P.r;
    G.transpose = 0;
    G.part = (float*)(wsb + pl.pb_off[p]);
    G.n = 1;
    G.G[0] = P.dB;
    G.r[0] = P.r;
    G.scale[0] = P.scale;
  }
  if ((e = launch_grad_jobs(gj, ng, (int)T, accumulate, s)) != hipSuccess) return hip_fail(e, "dA / dB launch");
  return LNF4_OK;
}

}  // namespace lnf4

using namespace lnf4;

// =========================================================================== extern "C"
extern "C" {

const char* lnf4_last_error(void) { return g_err.c_str(); }

const char* lnf4_version(void) { return "lnf4 0.1 gfx950"; }

int lnf4_nf4_table(float out[16]) {
  if (!out) return fail(LNF4_EINVAL, "lnf4_nf4_table: out is NULL");
  std::memcpy(out, kTable, sizeof kTable);
  return LNF4_OK;
}

int nf4_dequant(const uint8_t* codes, const float* absmax, int64_t n_elems, int32_t blocksize, uint16_t* out_bf16,
                hipStream_t stream) {
  const char* who = "nf4_dequant";
  if (blocksize != 64) return fail(LNF4_ESHAPE, "%s: blocksize=%d (only 64 is supported)", who, (int)blocksize);
  if (n_elems < 0 || n_elems % 64 != 0) return fail(LNF4_ESHAPE, "%s: n_elems=%lld not a non-negative multiple of 64", who, (long long)n_elems);
  if (n_elems == 0) return LNF4_OK;
  if (!codes || !absmax || !out_bf16) return fail(LNF4_EINVAL, "%s: NULL pointer", who);
  if (!aligned(codes, 16) || !aligned(out_bf16, 16) || !aligned(absmax, 4)) return fail(LNF4_EALIGN, "%s: misaligned pointer", who);
  hipError_t e = launch_nf4_dequant(codes, absmax, n_elems, out_bf16, stream);
  return e == hipSuccess ? LNF4_OK : hip_fail(e, "nf4_dequant launch");
}

int nf4_quantize(const float* w, int64_t n_elems, int32_t blocksize, uint8_t* codes, float* absmax, hipStream_t stream) {
  const char* who = "nf4_quantize";
  if (blocksize != 64) return fail(LNF4_ESHAPE, "%s: blocksize=%d (only 64 is supported)", who, (int)blocksize);
  if (n_elems < 0 || n_elems % 64 != 0) return fail(LNF4_ESHAPE, "%s: n_elems=%lld not a non-negative multiple of 64", who, (long long)n_elems);
  if (n_elems == 0) return LNF4_OK;
  if (!w || !codes || !absmax) return fail(LNF4_EINVAL, "%s: NULL pointer", who);
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(absmax, 4)) return fail(LNF4_EALIGN, "%s: misaligned pointer", who);
  hipError_t e = launch_nf4_quantize(w, n_elems, codes, absmax, stream);
  return e == hipSuccess ? LNF4_OK : hip_fail(e, "nf4_quantize launch");
}

int lora_linear_fwd(const lnf4_weight* W, const uint16_t* x, int64_t T, const uint16_t* A, const uint16_t* B, int32_t r,
                    float scale, uint16_t* y, float* u, hipStream_t stream) {
  if (!W) return fail(LNF4_EINVAL, "lora_linear_fwd: weight descriptor is NULL");
  lnf4_proj p;
  std::memset(&p, 0, sizeof p);
  p.W = *W;
  p.A = A;
  p.B = B;
  p.r = r;
  p.scale = scale;
  p.y = y;
  p.u = u;
  return group_fwd_impl(&p, 1, x, T, 1, nullptr, 0, stream, "lora_linear_fwd");
}

size_t lora_linear_bwd_workspace(int64_t T, int64_t out_f, int64_t in_f, int32_t r) {
  if (T < 0 || out_f < 1 || in_f < 1 || r < 0 || r > LNF4_MAX_RANK) return 0;
  lnf4_proj p;
  std::memset(&p, 0, sizeof p);
  p.W.out_f = out_f;
  p.W.in_f = in_f;
  p.r = r;
  // worst case: adapter on, both gradients asked for and u recomputed
  p.A = (const uint16_t*)16;
  p.B = (const uint16_t*)16;
  p.dA = (float*)16;
  p.dB = (float*)16;
  return group_bwd_ws(&p, 1, T);
}

int lora_linear_bwd(const lnf4_weight* W, const uint16_t* x, const uint16_t* dy, int64_t T, const uint16_t* A,
                    const uint16_t* B, int32_t r, float scale, const float* u_saved, uint16_t* dx, float* dA, float* dB,
                    int32_t accumulate, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!W) return fail(LNF4_EINVAL, "lora_linear_bwd: weight descriptor is NULL");
  lnf4_proj p;
  std::memset(&p, 0, sizeof p);
  p.W = *W;
  p.A = A;
  p.B = B;
  p.r = r;
  p.scale = scale;
  p.u = const_cast<float*>(u_saved);
  p.dy = dy;
  p.dA = dA;
  p.dB = dB;
  return group_bwd_impl(&p, 1, x, T, dx, accumulate, workspace, ws_bytes, stream, "lora_linear_bwd");
}

int lora_linear_bwd_noalloc(const lnf4_weight* W, const uint16_t* x, const uint16_t* dy, int64_t T,
                            const uint16_t* A, const uint16_t* B, int32_t r, float scale, const float* u_saved,
                            uint16_t* dx, float* dA, float* dB, int32_t accumulate, hipStream_t stream) {
  if (!W) return fail(LNF4_EINVAL, "lora_linear_bwd_noalloc: weight descriptor is NULL");
  lnf4_proj p;
  std::memset(&p, 0, sizeof p);
  p.W = *W;
  p.A = A;
  p.B = B;
  p.r = r;
  p.scale = scale;
  p.u = const_cast<float*>(u_saved);
  p.dy = dy;
  p.dA = dA;
  p.dB = dB;
  return group_bwd_impl(&p, 1, x, T, dx, accumulate, nullptr, 0, stream, "lora_linear_bwd_noalloc", true);
}

int lora_group_fwd(const lnf4_proj* projs, int32_t n, const uint16_t* x, int64_t T, int32_t adapters_enabled,
                   hipStream_t stream) {
  return group_fwd_impl(projs, n, x, T, adapters_enabled, nullptr, 0, stream, "lora_group_fwd");
}

size_t lora_group_fwd_workspace(const lnf4_proj* projs, int32_t n, int64_t T) { return group_fwd_ws(projs, n, T); }

int lora_group_fwd_ws(const lnf4_proj* projs, int32_t n, const uint16_t* x, int64_t T, int32_t adapters_enabled,
                      void* workspace, size_t ws_bytes, hipStream_t stream) {
  return group_fwd_impl(projs, n, x, T, adapters_enabled, workspace, ws_bytes, stream, "lora_group_fwd_ws");
}

size_t lora_group_bwd_workspace(const lnf4_proj* projs, int32_t n, int64_t T) { return group_bwd_ws(projs, n, T); }

int lora_group_bwd(const lnf4_proj* projs, int32_t n, const uint16_t* x, int64_t T, uint16_t* dx, int32_t accumulate,
                   void* workspace, size_t ws_bytes, hipStream_t stream) {
  return group_bwd_impl(projs, n, x, T, dx, accumulate, workspace, ws_bytes, stream, "lora_group_bwd");
}

int lnf4_shard_layout(int32_t n_proj, const int64_t* out_f, const int64_t* in_f, int32_t fmt, int64_t* offsets,
                      int64_t* total_bytes) {
  const char* who = "lnf4_shard_layout";
  if (n_proj < 1 || n_proj > 64) return fail(LNF4_EINVAL, "%s: n_proj=%d outside 1..64", who, (int)n_proj);
  if (!out_f || !in_f || !offsets || !total_bytes) return fail(LNF4_EINVAL, "%s: NULL pointer", who);
  if (fmt != LNF4_FMT_NF4 && fmt != LNF4_FMT_BF16) return fail(LNF4_EINVAL, "%s: unknown format %d", who, (int)fmt);
  int64_t off = 0;
  for (int p = 0; p < n_proj; ++p) {
    if (out_f[p] < 1 || in_f[p] < 64 || in_f[p] % 64 != 0)
      return fail(LNF4_ESHAPE, "%s: projection %d has shape %lldx%lld (in must be a positive multiple of 64)", who, p,
                  (long long)out_f[p], (long long)in_f[p]);
    const int64_t n = out_f[p] * in_f[p];
    offsets[2 * p] = off;
    if (fmt == LNF4_FMT_NF4) {
      off = (int64_t)round256((size_t)(off + n / 2));
      offsets[2 * p + 1] = off;
      off = (int64_t)round256((size_t)(off + (n / 64) * 4));
    } else {
      offsets[2 * p + 1] = -1;
      off = (int64_t)round256((size_t)(off + n * 2));
    }
  }
  *total_bytes = off;
  return LNF4_OK;
}

}  // extern "C"
