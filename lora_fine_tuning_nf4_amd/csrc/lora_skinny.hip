// Skinny rank-r LoRA products with wavefront-level reductions (no padded MFMA tiles).
//
//   u  = x  A^T   [T, r]   (forward; also the recompute when u was not saved)
//   v  = dy B     [T, r]   (first step of the backward)
//   dA = s v^T x  [r, in]  (reduction over T)
//   dB = s dy^T u [out, r] (reduction over T)
//
// u and v: one wavefront owns a few rows; its 64 lanes split the long dimension into
// 8-element chunks (16-byte loads), accumulate rows x rank partial sums, and finish with
// a butterfly reduce-scatter across the wave: at each xor-shuffle step a lane keeps half
// of its values and sends the other half, so 32 values need 16+8+4+2+1 shuffles plus one
// final pairwise add instead of 32 full reductions, and each lane ends up owning one
// finished value.  Results are fp32.
//
// dA and dB: each lane owns COLS columns and all r ranks; a workgroup covers a fixed slice
// of T; partial sums go to a workspace and a second kernel adds the slices in a fixed
// order (deterministic, no atomics).
#include "common.hpp"
#include "kernels.hpp"

namespace lnf4 {

template <int NV>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[NV], int lane) {
  // returns the total of value index (NV == 64 ? lane : lane >> 1)
#pragma unroll
  for (int w = NV / 2, mask = 32; w >= 1; w >>= 1, mask >>= 1) {
    const bool up = (lane & mask) != 0;
#pragma unroll
    for (int i = 0; i < w; ++i) {
      const float send = up ? v[i] : v[i + w];
      const float keep = up ? v[i + w] : v[i];
      v[i] = keep + __shfl_xor(send, mask, 64);
    }
  }
  float t = v[0];
  if (NV == 32) t += __shfl_xor(t, 1, 64);
  return t;
}

__device__ __forceinline__ void unpack8(const uint4& q, float f[8]) {
  f[0] = bf16_lo(q.x); f[1] = bf16_hi(q.x);
  f[2] = bf16_lo(q.y); f[3] = bf16_hi(q.y);
  f[4] = bf16_lo(q.z); f[5] = bf16_hi(q.z);
  f[6] = bf16_lo(q.w); f[7] = bf16_hi(q.w);
}

// ---------------------------------------------------------------- u = x A^T
// RMAX: rank capacity (r <= RMAX); RPW rows per wave, RPW * RMAX in {32, 64}.
template <int RMAX, int RPW>
__global__ __launch_bounds__(256) void k_xa(const uint16_t* __restrict__ x, const uint16_t* __restrict__ A,
                                            int T, int in_f, int r, float* __restrict__ u) {
  constexpr int NV = RPW * RMAX;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = (blockIdx.x * 4 + wave) * RPW;
  if (t0 >= T) return;  // whole wave exits together
  float acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.f;
  const int nch = in_f / 8;
  for (int c = lane; c < nch; c += 64) {
    float xf[RPW][8];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int t = (t0 + rr < T) ? t0 + rr : T - 1;
      unpack8(*(const uint4*)(x + (size_t)t * in_f + 8 * c), xf[rr]);
    }
#pragma unroll
    for (int k = 0; k < RMAX; ++k) {
      if (k < r) {
        float af[8];
        unpack8(*(const uint4*)(A + (size_t)k * in_f + 8 * c), af);
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
          float s = acc[rr * RMAX + k];
#pragma unroll
          for (int e = 0; e < 8; ++e) s += xf[rr][e] * af[e];
          acc[rr * RMAX + k] = s;
        }
      }
    }
  }
  const float tot = wave_reduce_scatter<NV>(acc, lane);
  const int idx = (NV == 64) ? lane : (lane >> 1);
  const int rr = idx / RMAX, k = idx % RMAX;
  const bool writer = (NV == 64) || ((lane & 1) == 0);
  if (writer && k < r && t0 + rr < T) u[(size_t)(t0 + rr) * r + k] = tot;
}

// ---------------------------------------------------------------- v = dy B
template <int RMAX, int RPW>
__global__ __launch_bounds__(256) void k_dyb(const uint16_t* __restrict__ dy, const uint16_t* __restrict__ B,
                                             int T, int out_f, int r, float* __restrict__ v) {
  constexpr int NV = RPW * RMAX;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = (blockIdx.x * 4 + wave) * RPW;
  if (t0 >= T) return;
  float acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.f;
  const int nch = out_f / 8;
  const bool fast = (r == RMAX);
  for (int c = lane; c < nch; c += 64) {
    float df[RPW][8];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int t = (t0 + rr < T) ? t0 + rr : T - 1;
      unpack8(*(const uint4*)(dy + (size_t)t * out_f + 8 * c), df[rr]);
    }
    // rows 8c .. 8c+7 of B, each r bf16
    const uint16_t* bp = B + (size_t)(8 * c) * r;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float bf[RMAX];
      if (fast) {
#pragma unroll
        for (int k8 = 0; k8 < RMAX / 8; ++k8) unpack8(*(const uint4*)(bp + e * RMAX + 8 * k8), bf + 8 * k8);
      } else {
#pragma unroll
        for (int k = 0; k < RMAX; ++k) bf[k] = (k < r) ? bf16_to_f32(bp[e * r + k]) : 0.f;
      }
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
        for (int k = 0; k < RMAX; ++k) acc[rr * RMAX + k] += df[rr][e] * bf[k];
    }
  }
  const float tot = wave_reduce_scatter<NV>(acc, lane);
  const int idx = (NV == 64) ? lane : (lane >> 1);
  const int rr = idx / RMAX, k = idx % RMAX;
  const bool writer = (NV == 64) || ((lane & 1) == 0);
  if (writer && k < r && t0 + rr < T) v[(size_t)(t0 + rr) * r + k] = tot;
}

// ---------------------------------------------------------------- dA / dB partials
static inline int grad_nsplit(int T) {
  int ns = (T + 63) / 64;
  return ns < 1 ? 1 : (ns > 32 ? 32 : ns);
}

template <int RMAX, int COLS>
__global__ __launch_bounds__(64) void k_grad_partial(const float* __restrict__ P, const uint16_t* __restrict__ Q,
                                                     int T, int C, int r, int tchunk, float* __restrict__ part) {
  const int lane = threadIdx.x;
  const int c0 = (blockIdx.x * 64 + lane) * COLS;
  const int split = blockIdx.y;
  const int tb = split * tchunk;
  const int te = (tb + tchunk < T) ? tb + tchunk : T;
  float acc[COLS][RMAX];
#pragma unroll
  for (int e = 0; e < COLS; ++e)
#pragma unroll
    for (int k = 0; k < RMAX; ++k) acc[e][k] = 0.f;
  const bool ok = c0 < C;
  const int cc = ok ? c0 : 0;
  for (int t = tb; t < te; ++t) {
    float q[COLS];
    if (COLS == 2) {
      const uint32_t w = *(const uint32_t*)(Q + (size_t)t * C + cc);
      q[0] = bf16_lo(w);
      q[COLS - 1] = bf16_hi(w);
    } else {
      q[0] = bf16_to_f32(Q[(size_t)t * C + cc]);
    }
    const float* pr = P + (size_t)t * r;
#pragma unroll
    for (int k = 0; k < RMAX; ++k) {
      const float pk = (k < r) ? pr[k] : 0.f;
#pragma unroll
      for (int e = 0; e < COLS; ++e) acc[e][k] += pk * q[e];
    }
  }
  if (!ok) return;
  float* dst = part + ((size_t)split * C + c0) * r;
#pragma unroll
  for (int e = 0; e < COLS; ++e)
#pragma unroll
    for (int k = 0; k < RMAX; ++k)
      if (k < r) dst[e * r + k] = acc[e][k];
}

__global__ __launch_bounds__(256) void k_grad_reduce(const float* __restrict__ part, int nsplit, int C, int r,
                                                     float scale, int transpose_out, int accumulate,
                                                     float* __restrict__ G) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // over C * r in [c][k] order
  const int64_t n = (int64_t)C * r;
  if (idx >= n) return;
  float s = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) s += part[(size_t)sp * n + idx];
  s *= scale;
  const int c = (int)(idx / r), k = (int)(idx % r);
  const size_t o = transpose_out ? (size_t)k * C + c : (size_t)idx;
  G[o] = accumulate ? G[o] + s : s;
}

__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// ---------------------------------------------------------------- launchers
// Zero-fill with a kernel rather than a memset node, so the call is safe to capture.
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_xa(const uint16_t* x, const uint16_t* A, int32_t T, int32_t in_f, int32_t r, float* u,
                     hipStream_t s) {
  if (T <= 0 || r <= 0) return hipSuccess;
  const dim3 blk(256);
  if (r <= 8) hipLaunchKernelGGL((k_xa<8, 4>), dim3((T + 15) / 16), blk, 0, s, x, A, T, in_f, r, u);
  else if (r <= 16) hipLaunchKernelGGL((k_xa<16, 2>), dim3((T + 7) / 8), blk, 0, s, x, A, T, in_f, r, u);
  else if (r <= 32) hipLaunchKernelGGL((k_xa<32, 1>), dim3((T + 3) / 4), blk, 0, s, x, A, T, in_f, r, u);
  else hipLaunchKernelGGL((k_xa<64, 1>), dim3((T + 3) / 4), blk, 0, s, x, A, T, in_f, r, u);
  return hipGetLastError();
}

hipError_t launch_dyb(const uint16_t* dy, const uint16_t* B, int32_t T, int32_t out_f, int32_t r, float* v,
                      hipStream_t s) {
  if (T <= 0 || r <= 0) return hipSuccess;
  const dim3 blk(256);
  if (r <= 8) hipLaunchKernelGGL((k_dyb<8, 4>), dim3((T + 15) / 16), blk, 0, s, dy, B, T, out_f, r, v);
  else if (r <= 16) hipLaunchKernelGGL((k_dyb<16, 2>), dim3((T + 7) / 8), blk, 0, s, dy, B, T, out_f, r, v);
  else if (r <= 32) hipLaunchKernelGGL((k_dyb<32, 1>), dim3((T + 3) / 4), blk, 0, s, dy, B, T, out_f, r, v);
  else hipLaunchKernelGGL((k_dyb<64, 1>), dim3((T + 3) / 4), blk, 0, s, dy, B, T, out_f, r, v);
  return hipGetLastError();
}

size_t grad_workspace_bytes(int32_t T, int32_t C, int32_t r) {
  if (T <= 0 || r <= 0 || C <= 0) return 0;
  return (size_t)grad_nsplit(T) * (size_t)C * (size_t)r * sizeof(float);
}

hipError_t launch_grad(const float* P, const uint16_t* Q, int32_t T, int32_t C, int32_t r, float scale,
                       int32_t transpose_out, int32_t accumulate, float* G, float* partial, hipStream_t s) {
  if (r <= 0 || C <= 0) return hipSuccess;
  if (T <= 0) {
    // empty reduction: the gradient is zero (or unchanged when accumulating)
    if (!accumulate) return launch_fill_zero(G, (int64_t)C * r, s);
    return hipSuccess;
  }
  const int ns = grad_nsplit(T);
  const int tchunk = (T + ns - 1) / ns;
  if (r <= 8) {
    const dim3 grid((C + 127) / 128, ns);
    hipLaunchKernelGGL((k_grad_partial<8, 2>), grid, dim3(64), 0, s, P, Q, T, C, r, tchunk, partial);
  } else if (r <= 16) {
    const dim3 grid((C + 127) / 128, ns);
    hipLaunchKernelGGL((k_grad_partial<16, 2>), grid, dim3(64), 0, s, P, Q, T, C, r, tchunk, partial);
  } else if (r <= 32) {
    const dim3 grid((C + 63) / 64, ns);
    hipLaunchKernelGGL((k_grad_partial<32, 1>), grid, dim3(64), 0, s, P, Q, T, C, r, tchunk, partial);
  } else {
    const dim3 grid((C + 63) / 64, ns);
    hipLaunchKernelGGL((k_grad_partial<64, 1>), grid, dim3(64), 0, s, P, Q, T, C, r, tchunk, partial);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)C * r;
  hipLaunchKernelGGL(k_grad_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, partial, ns, C, r, scale,
                     transpose_out, accumulate, G);
  return hipGetLastError();
}

}  // namespace lnf4
