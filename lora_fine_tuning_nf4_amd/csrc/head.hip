// Output side of a streamed step: embedding gather from the head slot, token
// cross-entropy on the untied head's bf16 logits (log-prob of each label and the logit
// gradient), fixed-order sequence sums, and the sigmoid preference loss.
//
// Cross-entropy: one workgroup per token row.  Each thread keeps an online (max, sum of
// exp) pair over a fixed stride of the row (16-byte loads), the pairs merge in a fixed
// tree through LDS into the row's log-sum-exp, and a second pass writes
// dlogits = g_t * (softmax - onehot) rounded to bf16.  Every reduction has a fixed
// order, so results are bitwise reproducible.
#include <math.h>

#include "common.hpp"
#include "head.hpp"

namespace lnf4 {

// ------------------------------------------------------------------ embedding gather
// out[t][8c .. 8c+7] = table[ids[t]][8c .. 8c+7]; ids outside [0, vocab) give zero rows.
// One workgroup per row (rows beyond the grid are taken by a stride loop), one 16-byte
// chunk per lane.
__global__ __launch_bounds__(256) void k_embed_gather(const uint16_t* __restrict__ table, int64_t vocab,
                                                      int64_t hidden, const int32_t* __restrict__ ids, int64_t T,
                                                      uint16_t* __restrict__ out) {
  const int64_t nch = hidden / 8;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const int32_t id = ids[t];
    const bool ok = id >= 0 && (int64_t)id < vocab;
    const uint16_t* src = table + (size_t)(ok ? id : 0) * hidden;
    uint16_t* dst = out + (size_t)t * hidden;
    for (int64_t c = threadIdx.x; c < nch; c += 256) {
      u32x4 v = u32x4{0, 0, 0, 0};
      if (ok) v = *(const u32x4*)(src + 8 * c);
      *(u32x4*)(dst + 8 * c) = v;
    }
  }
}

// ------------------------------------------------------------------ cross-entropy
// Running (max, sum of exp(x - max)) pair; an empty pair is (-inf, 0).
struct MaxSum {
  float m, s;
};

__device__ __forceinline__ MaxSum ms_merge(MaxSum a, MaxSum b) {
  if (b.m > a.m) {
    const MaxSum t = a;
    a = b;
    b = t;
  }
  if (b.s > 0.0f) a.s += b.s * expf(b.m - a.m);  // a.m >= b.m
  return a;
}

// A label outside [0, V) marks an ignored token: log-prob 0 and a zero gradient row.
// dlogits may alias logits: each thread rewrites only the chunks it has just read.
__global__ __launch_bounds__(256) void k_cross_entropy(const uint16_t* logits, int64_t T, int64_t V,
                                                       const int32_t* __restrict__ labels, float grad_scale,
                                                       const float* __restrict__ seq_scale, int64_t rows_per_scale,
                                                       float* __restrict__ logp, uint16_t* dlogits) {
  __shared__ float sm_m[256], sm_s[256];
  const int tid = threadIdx.x;
  const int64_t nch = V / 8;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const uint16_t* row = logits + (size_t)t * V;
    const int32_t lab = labels[t];
    const bool lab_ok = lab >= 0 && (int64_t)lab < V;
    // read before the barriers below: dlogits may overwrite the row in place
    const float lab_logit = (tid == 0 && lab_ok) ? bf16_to_f32(row[lab]) : 0.0f;

    // pass 1: per-lane running (max, sum) over chunks tid, tid+256, ...; one rescale per chunk
    MaxSum a{-INFINITY, 0.0f};
    for (int64_t c = tid; c < nch; c += 256) {
      const u32x4 q = *(const u32x4*)(row + 8 * c);
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_lo(q[i]);
        f[2 * i + 1] = bf16_hi(q[i]);
      }
      float m8 = f[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) m8 = fmaxf(m8, f[e]);
      if (m8 > a.m) {
        a.s *= expf(a.m - m8);
        a.m = m8;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) a.s += expf(f[e] - a.m);
    }
    sm_m[tid] = a.m;
    sm_s[tid] = a.s;
    __syncthreads();
#pragma unroll
    for (int w = 128; w >= 1; w >>= 1) {
      if (tid < w) {
        const MaxSum r = ms_merge(MaxSum{sm_m[tid], sm_s[tid]}, MaxSum{sm_m[tid + w], sm_s[tid + w]});
        sm_m[tid] = r.m;
        sm_s[tid] = r.s;
      }
      __syncthreads();
    }
    const float lse = sm_m[0] + logf(sm_s[0]);
    __syncthreads();  // every lane has read the row's result before the next row reuses LDS
    if (tid == 0 && logp != nullptr) logp[t] = lab_ok ? lab_logit - lse : 0.0f;
    if (dlogits == nullptr) continue;

    // pass 2: g_t * (softmax - onehot), rounded to bf16
    const float g = lab_ok ? grad_scale * (seq_scale != nullptr ? seq_scale[t / rows_per_scale] : 1.0f) : 0.0f;
    uint16_t* drow = dlogits + (size_t)t * V;
    for (int64_t c = tid; c < nch; c += 256) {
      const u32x4 q = *(const u32x4*)(row + 8 * c);
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t j0 = 8 * c + 2 * i;
        float p0 = expf(bf16_lo(q[i]) - lse), p1 = expf(bf16_hi(q[i]) - lse);
        if (j0 == lab) p0 -= 1.0f;
        if (j0 + 1 == lab) p1 -= 1.0f;
        o[i] = lab_ok ? pack_bf16x2(g * p0, g * p1) : 0u;  // +0 bits for an ignored row
      }
      *(u32x4*)(drow + 8 * c) = o;
    }
  }
}

// ------------------------------------------------------------------ sequence sums
// sums[i] = x[i*L] + ... + x[i*L + L-1]: 256 threads take a fixed stride each, then a
// fixed tree.
__global__ __launch_bounds__(256) void k_sequence_sums(const float* __restrict__ x, int64_t n_seq, int64_t L,
                                                       float* __restrict__ sums) {
  __shared__ float sm[256];
  const int tid = threadIdx.x;
  for (int64_t i = blockIdx.x; i < n_seq; i += gridDim.x) {
    float s = 0.0f;
    for (int64_t j = tid; j < L; j += 256) s += x[i * L + j];
    sm[tid] = s;
    __syncthreads();
#pragma unroll
    for (int w = 128; w >= 1; w >>= 1) {
      if (tid < w) sm[tid] += sm[tid + w];
      __syncthreads();
    }
    if (tid == 0) sums[i] = sm[0];
    __syncthreads();
  }
}

// ------------------------------------------------------------------ sigmoid DPO
// margins m_p = beta ((pol_c - ref_c) - (pol_r - ref_r)); loss = mean_p softplus(-m_p);
// coef = dL/dpol: (-beta sigmoid(-m_p) / P, +beta sigmoid(-m_p) / P) per pair.  One
// thread walks the pairs in order (P is a handful).
__global__ void k_dpo_loss(const float* __restrict__ pol, const float* __restrict__ ref, int P, float beta,
                           float* __restrict__ loss, float* __restrict__ coef) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  float acc = 0.0f;
  for (int p = 0; p < P; ++p) {
    const float m = beta * ((pol[2 * p] - ref[2 * p]) - (pol[2 * p + 1] - ref[2 * p + 1]));
    acc += fmaxf(-m, 0.0f) + log1pf(expf(-fabsf(m)));    // softplus(-m)
    const float sn = 1.0f / (1.0f + expf(m));             // sigmoid(-m)
    coef[2 * p] = -beta * sn / (float)P;
    coef[2 * p + 1] = beta * sn / (float)P;
  }
  *loss = acc / (float)P;
}

// ------------------------------------------------------------------ launchers
// one workgroup per row up to 64 Ki rows; beyond that the kernels' stride loops take over
static unsigned grid_rows(int64_t rows) { return (unsigned)(rows < 65536 ? rows : 65536); }

hipError_t launch_embed_gather(const uint16_t* table, int64_t vocab, int64_t hidden, const int32_t* ids, int64_t T,
                               uint16_t* out, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_embed_gather, dim3(grid_rows(T)), dim3(256), 0, s, table, vocab, hidden, ids, T, out);
  return hipGetLastError();
}

hipError_t launch_cross_entropy(const uint16_t* logits, int64_t T, int64_t V, const int32_t* labels, float grad_scale,
                                const float* seq_scale, int64_t rows_per_scale, float* logp, uint16_t* dlogits,
                                hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_cross_entropy, dim3(grid_rows(T)), dim3(256), 0, s, logits, T, V, labels, grad_scale,
                     seq_scale, rows_per_scale, logp, dlogits);
  return hipGetLastError();
}

hipError_t launch_sequence_sums(const float* x, int32_t n_seq, int64_t L, float* sums, hipStream_t s) {
  if (n_seq <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_sequence_sums, dim3(grid_rows(n_seq)), dim3(256), 0, s, x, (int64_t)n_seq, L, sums);
  return hipGetLastError();
}

hipError_t launch_dpo_loss(const float* pol, const float* ref, int32_t P, float beta, float* loss, float* coef,
                           hipStream_t s) {
  hipLaunchKernelGGL(k_dpo_loss, dim3(1), dim3(64), 0, s, pol, ref, (int)P, beta, loss, coef);
  return hipGetLastError();
}

}  // namespace lnf4
