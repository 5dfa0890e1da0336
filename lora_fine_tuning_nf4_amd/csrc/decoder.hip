// The glue of a decoder layer between its projections: RMSNorm (forward and backward,
// the backward adding the residual gradient), rotate-half RoPE from a per-position
// cos/sin table, SwiGLU (forward and backward) and the residual add.  All of it is
// HBM-bound elementwise or row work: 16-byte vector accesses, one workgroup per row
// for the row reductions (fixed order: bitwise reproducible), fp32 arithmetic and one
// bf16 rounding per stored value.
#include <math.h>

#include "common.hpp"
#include "decoder.hpp"

namespace lnf4 {

namespace {

__device__ __forceinline__ void unpack8(const u32x4 q, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(q[i]);
    f[2 * i + 1] = bf16_hi(q[i]);
  }
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  u32x4 q;
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return q;
}

// fixed-order sum of one value per thread over a 256-thread workgroup (LDS tree)
__device__ __forceinline__ float block_sum256(float v, float* sm) {
  const int tid = threadIdx.x;
  sm[tid] = v;
  __syncthreads();
#pragma unroll
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) sm[tid] += sm[tid + w];
    __syncthreads();
  }
  const float r = sm[0];
  __syncthreads();
  return r;
}

unsigned grid_rows(int64_t rows) { return (unsigned)(rows < 65536 ? rows : 65536); }

}  // namespace

// ------------------------------------------------------------------ RMSNorm
// y = bf16(x * r * g), r = 1/sqrt(mean(x^2) + eps) (fp32), rstd[t] = r.
__global__ __launch_bounds__(256) void k_rmsnorm_fwd(const uint16_t* __restrict__ x, int64_t T, int64_t H,
                                                     const uint16_t* __restrict__ g, float eps,
                                                     uint16_t* __restrict__ y, float* __restrict__ rstd) {
  __shared__ float sm[256];
  const int64_t nch = H / 8;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const uint16_t* xr = x + (size_t)t * H;
    float ss = 0.0f;
    for (int64_t c = threadIdx.x; c < nch; c += 256) {
      float f[8];
      unpack8(*(const u32x4*)(xr + 8 * c), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
    }
    const float r = 1.0f / sqrtf(block_sum256(ss, sm) / (float)H + eps);
    if (threadIdx.x == 0 && rstd != nullptr) rstd[t] = r;
    uint16_t* yr = y + (size_t)t * H;
    for (int64_t c = threadIdx.x; c < nch; c += 256) {
      float f[8], w[8];
      unpack8(*(const u32x4*)(xr + 8 * c), f);
      unpack8(*(const u32x4*)(g + 8 * c), w);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = f[e] * r * w[e];
      *(u32x4*)(yr + 8 * c) = pack8(f);
    }
  }
}

// dx = bf16(dres + r g dy - x r^3 mean(x g dy)); r from the forward (rstd).
__global__ __launch_bounds__(256) void k_rmsnorm_bwd(const uint16_t* __restrict__ x, int64_t T, int64_t H,
                                                     const uint16_t* __restrict__ g, const float* __restrict__ rstd,
                                                     const uint16_t* __restrict__ dy,
                                                     const uint16_t* __restrict__ dres, uint16_t* __restrict__ dx) {
  __shared__ float sm[256];
  const int64_t nch = H / 8;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const uint16_t* xr = x + (size_t)t * H;
    const uint16_t* dyr = dy + (size_t)t * H;
    float dot = 0.0f;
    for (int64_t c = threadIdx.x; c < nch; c += 256) {
      float f[8], w[8], d[8];
      unpack8(*(const u32x4*)(xr + 8 * c), f);
      unpack8(*(const u32x4*)(g + 8 * c), w);
      unpack8(*(const u32x4*)(dyr + 8 * c), d);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += f[e] * (w[e] * d[e]);
    }
    const float r = rstd[t];
    const float k = r * r * r * (block_sum256(dot, sm) / (float)H);
    uint16_t* dxr = dx + (size_t)t * H;
    for (int64_t c = threadIdx.x; c < nch; c += 256) {
      float f[8], w[8], d[8], o[8];
      unpack8(*(const u32x4*)(xr + 8 * c), f);
      unpack8(*(const u32x4*)(g + 8 * c), w);
      unpack8(*(const u32x4*)(dyr + 8 * c), d);
      if (dres != nullptr) unpack8(*(const u32x4*)(dres + (size_t)t * H + 8 * c), o);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = r * (w[e] * d[e]) - f[e] * k;
        o[e] = dres != nullptr ? o[e] + v : v;
      }
      *(u32x4*)(dxr + 8 * c) = pack8(o);
    }
  }
}

// ------------------------------------------------------------------ RoPE
// table[p][i] = (cos, sin)(p * base^(-2i/D)), computed in fp64 and rounded to fp32.
__global__ void k_rope_table(int64_t seq_len, int D, double log2_base, float2* __restrict__ table) {
  const int64_t n = seq_len * (D / 2);
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = idx / (D / 2);
    const int i = (int)(idx - p * (D / 2));
    const double inv = exp2(-(2.0 * i / D) * log2_base);
    const double a = (double)p * inv;
    table[idx] = make_float2((float)cos(a), (float)sin(a));
  }
}

// In place on x [T, n_heads * D]: pairs (i, i + D/2) of every head turn by the angle of
// position t mod seq_len (by minus that angle when inverse).  A lane takes 8 pairs.
__global__ __launch_bounds__(256) void k_rope(uint16_t* __restrict__ x, int64_t T, int n_heads, int D,
                                              int64_t seq_len, const float2* __restrict__ table, int inverse) {
  const int half = D / 2, per_head = half / 8, lanes = n_heads * per_head;
  const int64_t ld = (int64_t)n_heads * D;
  const float sgn = inverse ? -1.0f : 1.0f;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const float2* tab = table + (t % seq_len) * half;
    for (int l = threadIdx.x; l < lanes; l += 256) {
      const int h = l / per_head, i0 = (l - h * per_head) * 8;
      uint16_t* pa = x + t * ld + (int64_t)h * D + i0;
      uint16_t* pb = pa + half;
      float a[8], b[8], oa[8], ob[8];
      unpack8(*(const u32x4*)pa, a);
      unpack8(*(const u32x4*)pb, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float2 cs = tab[i0 + e];
        const float s = sgn * cs.y;
        oa[e] = a[e] * cs.x - b[e] * s;
        ob[e] = b[e] * cs.x + a[e] * s;
      }
      *(u32x4*)pa = pack8(oa);
      *(u32x4*)pb = pack8(ob);
    }
  }
}

// ------------------------------------------------------------------ SwiGLU, residual
__global__ __launch_bounds__(256) void k_swiglu_fwd(const uint16_t* __restrict__ g, const uint16_t* __restrict__ u,
                                                    int64_t n8, uint16_t* __restrict__ s) {
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n8; c += (int64_t)gridDim.x * 256) {
    float a[8], b[8];
    unpack8(*(const u32x4*)(g + 8 * c), a);
    unpack8(*(const u32x4*)(u + 8 * c), b);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = a[e] / (1.0f + expf(-a[e])) * b[e];
    *(u32x4*)(s + 8 * c) = pack8(a);
  }
}

// dg = ds u sig (1 + g (1 - sig)), du = ds g sig, sig = 1 / (1 + e^-g)
__global__ __launch_bounds__(256) void k_swiglu_bwd(const uint16_t* __restrict__ g, const uint16_t* __restrict__ u,
                                                    const uint16_t* __restrict__ ds, int64_t n8,
                                                    uint16_t* __restrict__ dg, uint16_t* __restrict__ du) {
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n8; c += (int64_t)gridDim.x * 256) {
    float a[8], b[8], d[8], og[8], ou[8];
    unpack8(*(const u32x4*)(g + 8 * c), a);
    unpack8(*(const u32x4*)(u + 8 * c), b);
    unpack8(*(const u32x4*)(ds + 8 * c), d);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sig = 1.0f / (1.0f + expf(-a[e]));
      og[e] = d[e] * b[e] * sig * (1.0f + a[e] * (1.0f - sig));
      ou[e] = d[e] * a[e] * sig;
    }
    *(u32x4*)(dg + 8 * c) = pack8(og);
    *(u32x4*)(du + 8 * c) = pack8(ou);
  }
}

__global__ __launch_bounds__(256) void k_add(const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
                                             int64_t n8, uint16_t* __restrict__ out) {
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n8; c += (int64_t)gridDim.x * 256) {
    float p[8], q[8];
    unpack8(*(const u32x4*)(a + 8 * c), p);
    unpack8(*(const u32x4*)(b + 8 * c), q);
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] += q[e];
    *(u32x4*)(out + 8 * c) = pack8(p);
  }
}

// ------------------------------------------------------------------ launchers
static unsigned grid_elems(int64_t n8) {
  const int64_t b = (n8 + 255) / 256;
  return (unsigned)(b < 8192 ? (b > 0 ? b : 1) : 8192);
}

hipError_t launch_rmsnorm_fwd(const uint16_t* x, int64_t T, int64_t H, const uint16_t* g, float eps, uint16_t* y,
                              float* rstd, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rmsnorm_fwd, dim3(grid_rows(T)), dim3(256), 0, s, x, T, H, g, eps, y, rstd);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const uint16_t* x, int64_t T, int64_t H, const uint16_t* g, const float* rstd,
                              const uint16_t* dy, const uint16_t* dres, uint16_t* dx, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rmsnorm_bwd, dim3(grid_rows(T)), dim3(256), 0, s, x, T, H, g, rstd, dy, dres, dx);
  return hipGetLastError();
}

hipError_t launch_rope_table(int64_t seq_len, int D, double base, float2* table, hipStream_t s) {
  const int64_t n = seq_len * (D / 2);
  const int64_t b = (n + 255) / 256;
  hipLaunchKernelGGL(k_rope_table, dim3((unsigned)(b < 4096 ? b : 4096)), dim3(256), 0, s, seq_len, D, log2(base),
                     table);
  return hipGetLastError();
}

hipError_t launch_rope(uint16_t* x, int64_t T, int n_heads, int D, int64_t seq_len, const float2* table, int inverse,
                       hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rope, dim3(grid_rows(T)), dim3(256), 0, s, x, T, n_heads, D, seq_len, table, inverse);
  return hipGetLastError();
}

hipError_t launch_swiglu_fwd(const uint16_t* g, const uint16_t* u, int64_t n, uint16_t* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_swiglu_fwd, dim3(grid_elems(n / 8)), dim3(256), 0, s, g, u, n / 8, out);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const uint16_t* g, const uint16_t* u, const uint16_t* ds, int64_t n, uint16_t* dg,
                             uint16_t* du, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_swiglu_bwd, dim3(grid_elems(n / 8)), dim3(256), 0, s, g, u, ds, n / 8, dg, du);
  return hipGetLastError();
}

hipError_t launch_add(const uint16_t* a, const uint16_t* b, int64_t n, uint16_t* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_add, dim3(grid_elems(n / 8)), dim3(256), 0, s, a, b, n / 8, out);
  return hipGetLastError();
}

}  // namespace lnf4
