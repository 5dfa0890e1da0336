// Host-side launch interface of the lnf4 kernels.  Shapes are validated by the ABI layer
// before anything here is called; launchers only pick a configuration and launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lnf4 {

constexpr int kMaxGroup = 8;

// ---------------------------------------------------------------- fused forward GEMM
// y_p[T, out_p] = bf16( x[T, in] W'_p^T + scale_p * u_p B_p^T ) for the projections p of a
// group that share x.  W'_p is decoded from NF4 (or read as bf16) inside the kernel.
struct FwdProj {
  const void* w;        // NF4 codes [out][in/2] or bf16 [out][in]
  const float* absmax;  // NF4: [out*in/64]
  uint16_t* y;          // [T][out]
  const float* u;       // [T][r] fp32, or null (adapter off)
  const uint16_t* B;    // [out][r] bf16
  int32_t out_f;
  int32_t r;
  float scale;
  int32_t tile_n0;      // first N-tile of this projection in the group's tile space
};
struct FwdArgs {
  const uint16_t* x;
  int32_t M;            // T
  int32_t K;            // in
  int32_t n_proj;
  int32_t n_tiles_n;    // total N-tiles over the group
  int32_t n_tiles_m;
  FwdProj p[kMaxGroup];
};

// ---------------------------------------------------------------- fused dx GEMM
// dx[T, in] = bf16( sum_p dy_p W'_p + scale_p v_p A_p  (+ dx if accumulate) )
struct DxProj {
  const void* w;        // NF4 codes [out][in/2] or bf16 [out][in]
  const float* absmax;
  const uint16_t* dy;   // [T][out]
  const float* v;       // [T][r] fp32 or null
  const uint16_t* A;    // [r][in] bf16
  int32_t out_f;        // K extent of this projection (multiple of 8)
  int32_t r;
  float scale;
  int32_t kb0;          // first 64-wide K-block of this projection in the group's K space
};
struct DxArgs {
  uint16_t* dx;
  int32_t M;            // T
  int32_t N;            // in
  int32_t n_proj;
  int32_t total_kb;
  int32_t n_tiles_m;
  int32_t n_tiles_n;
  int32_t accumulate;
  DxProj p[kMaxGroup];
};

hipError_t launch_fwd(const FwdArgs& a, int fmt, hipStream_t s);
hipError_t launch_dx(const DxArgs& a, int fmt, hipStream_t s);

// ---------------------------------------------------------------- NF4 codec
hipError_t launch_nf4_dequant(const uint8_t* codes, const float* absmax, int64_t n_elems, uint16_t* out,
                              hipStream_t s);
hipError_t launch_nf4_quantize(const float* w, int64_t n_elems, uint8_t* codes, float* absmax,
                               hipStream_t s);

// ---------------------------------------------------------------- skinny LoRA products
// u[T][r] = x[T][in] A[r][in]^T            (fp32 out)
hipError_t launch_xa(const uint16_t* x, const uint16_t* A, int32_t T, int32_t in_f, int32_t r, float* u,
                     hipStream_t s);
// v[T][r] = dy[T][out] B[out][r]           (fp32 out)
hipError_t launch_dyb(const uint16_t* dy, const uint16_t* B, int32_t T, int32_t out_f, int32_t r, float* v,
                      hipStream_t s);
// G = scale * P^T Q over T with P [T][r] fp32 and Q [T][C] bf16:
//   transpose_out = 1: G is [r][C] (dA with P = v, Q = x)
//   transpose_out = 0: G is [C][r] (dB with P = u, Q = dy)
// Deterministic: fixed split over T into partials (workspace), fixed-order reduce.
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
size_t grad_workspace_bytes(int32_t T, int32_t C, int32_t r);
hipError_t launch_grad(const float* P, const uint16_t* Q, int32_t T, int32_t C, int32_t r, float scale,
                       int32_t transpose_out, int32_t accumulate, float* G, float* partial, hipStream_t s);

}  // namespace lnf4
