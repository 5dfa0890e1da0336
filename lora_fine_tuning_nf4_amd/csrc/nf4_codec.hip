// NF4 decode (the per-layer dequantization) and NF4 quantize (shard set-up) for gfx950.
//
// Decode is HBM-bound: per element it reads 0.5 B of code and 1/64 of a 4-byte scale
// and writes 2 B of bf16.  Each thread takes 32 consecutive elements: one 16-byte
// load of codes, one absmax (every 32-element run lies inside one 64-element block),
// four 16-byte stores.  Consecutive threads touch consecutive memory.
#include "common.hpp"
#include "kernels.hpp"

namespace lnf4 {

__constant__ float c_nf4_table[16] = LNF4_TABLE_INIT;

// Each wave takes 2048 consecutive elements (256 groups of 8) per trip: lane L decodes
// groups 64s + L (s = 0..3), so every load instruction reads 256 contiguous bytes of codes
// and every store writes 1 KB of contiguous output (whole lines; a lane writing 64 bytes of
// its own would spread each store over 64 partial lines).  The loads of a trip are all in
// flight before the first decode.
__global__ __launch_bounds__(256) void k_nf4_dequant(const uint32_t* __restrict__ codes,
                                                     const float* __restrict__ absmax,
                                                     uint4* __restrict__ out, int64_t n8) {
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = c_nf4_table[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t wv = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6; wv * 256 < n8; wv += nwaves) {
    uint32_t c[4];
    float a[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t g = wv * 256 + 64 * s + lane;  // group of 8 elements (4 code bytes)
      c[s] = g < n8 ? codes[g] : 0u;
      a[s] = g < n8 ? absmax[g >> 3] : 0.0f;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t g = wv * 256 + 64 * s + lane;
      if (g < n8) {
        uint32_t o[4];
        decode8(c[s], a[s], lut, o);
        out[g] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
}

hipError_t launch_nf4_dequant(const uint8_t* codes, const float* absmax, int64_t n_elems, uint16_t* out,
                              hipStream_t s) {
  const int64_t n8 = n_elems / 8;
  if (n8 == 0) return hipSuccess;
  int64_t blocks = (n8 + 1023) / 1024;  // 4 waves x 256 groups per trip
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(k_nf4_dequant, dim3((unsigned)blocks), dim3(256), 0, s, (const uint32_t*)codes, absmax,
                     (uint4*)out, n8);
  return hipGetLastError();
}

// One thread per 64-element block: absmax, then per element the nearest level of
// w / absmax (IEEE fp32 division, ties to the lower index), packed two per byte.
__global__ __launch_bounds__(256) void k_nf4_quantize(const float4* __restrict__ w, int64_t n_blocks,
                                                      uint4* __restrict__ codes, float* __restrict__ absmax) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= n_blocks) return;
  const float T[16] = LNF4_TABLE_INIT;
  float v[64];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const float4 f = w[b * 16 + q];
    v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
  }
  float am = 0.0f;
#pragma unroll
  for (int e = 0; e < 64; ++e) am = fmaxf(am, fabsf(v[e]));
  absmax[b] = am;
  uint32_t packed[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) packed[q] = 0;
#pragma unroll
  for (int e = 0; e < 64; ++e) {
    uint32_t code = 7;
    if (am > 0.0f) {
      const float x = v[e] / am;
      float best = fabsf(x - T[0]);
      code = 0;
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        const float d = fabsf(x - T[i]);
        if (d < best) { best = d; code = (uint32_t)i; }
      }
    }
    // element e -> byte e/2 (high nibble for even e); byte k sits at bits 8*(k%4) of dword k/4
    const int byte = e >> 1;
    const int shift = 8 * (byte & 3) + ((e & 1) ? 0 : 4);
    packed[byte >> 2] |= code << shift;
  }
  codes[b * 2] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  codes[b * 2 + 1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
}

hipError_t launch_nf4_quantize(const float* w, int64_t n_elems, uint8_t* codes, float* absmax,
                               hipStream_t s) {
  const int64_t nb = n_elems / 64;
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(k_nf4_quantize, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, (const float4*)w, nb,
                     (uint4*)codes, absmax);
  return hipGetLastError();
}

}  // namespace lnf4
