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
  int64_t part_off;     // K-split launches: this projection's fp32 sums [ksplit][T][out] at part + part_off
};
struct FwdArgs {
  const uint16_t* x;
  int32_t M;            // T
  int32_t K;            // in
  int32_t n_proj;
  int32_t n_tiles_n;    // N-tiles covered by this launch
  int32_t n_tiles_m;
  int32_t tn_base;      // first N-tile of this launch in the group's tile space
  // 128-row tail (set by launch_fwd): tail_m x tail_n tiles over the N-tiles that follow
  // n_tiles_n.  xcd_f == 0: blocks from split_block on run the tail.  xcd_f > 0: the XCD of
  // block b (b mod 8) takes xcd_f full and xcd_h tail tiles, XCDs 0-3 full tiles first,
  // XCDs 4-7 tail tiles first.
  int32_t split_block;
  int32_t tail_m;
  int32_t tail_n;
  int32_t xcd_f;
  int32_t xcd_h;
  // K splits (NF4, 128- and 64-row tiles; set by launch_fwd): ksplit > 1 runs every tile
  // ksplit times, split s over K-blocks [s kb_per_split, (s+1) kb_per_split), each writing
  // its fp32 sums to part; a second launch adds the splits in order into y
  int32_t ksplit;
  int32_t kb_per_split;
  float* part;
  FwdProj p[kMaxGroup];
};
// K splits of the forward: split count and workspace bytes (0: not split) for (T, the
// projections' out_f, in, fmt)
int fwd_split_count(int M, const int32_t* out_f, int n_proj, int K, int fmt);
size_t fwd_split_bytes(int M, const int32_t* out_f, int n_proj, int K, int fmt);

// ---------------------------------------------------------------- fused dx GEMM
// dx[T, in] = bf16( sum_p dy_p W'_p + scale_p v_p A_p  (+ dx if accumulate) )
struct DxProj {
  const void* w;        // NF4 codes [out][in/2] or bf16 [out][in]
  const float* absmax;
  const uint16_t* dy;   // [T][out]
  const float* v;       // [T][v_stride] fp32 (this projection's r columns) or null
  const uint16_t* A;    // [r][in] bf16
  int32_t out_f;        // K extent of this projection (multiple of 8)
  int32_t r;
  float scale;
  int32_t kb0;          // first 64-wide K-block of this projection in the group's K space
  int32_t v_stride;
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
  int32_t kb_per_split; // K-blocks per split (set by launch_dx)
  float* part;          // split-K workspace [splits][M][N] fp32 (dx_split_bytes), or null
  DxProj p[kMaxGroup];
};
// split-K of the input gradient: split count and workspace bytes for (T, in, K-blocks, fmt)
int dx_split_count(int M, int N, int total_kb, int fmt);
size_t dx_split_bytes(int M, int N, int total_kb, int fmt);

hipError_t launch_fwd(const FwdArgs& a, int fmt, hipStream_t s);
hipError_t launch_dx(const DxArgs& a, int fmt, hipStream_t s);

// ---------------------------------------------------------------- NF4 codec
hipError_t launch_nf4_dequant(const uint8_t* codes, const float* absmax, int64_t n_elems, uint16_t* out,
                              hipStream_t s);
hipError_t launch_nf4_quantize(const float* w, int64_t n_elems, uint8_t* codes, float* absmax,
                               hipStream_t s);

// ---------------------------------------------------------------- skinny LoRA products
constexpr int kMaxJobs = 8;
// One activation matrix src [T][K] bf16 times the weights of one job, ranks concatenated
// (R = sum r_p <= 64):
//   layout 0: W_p = A_p [r_p][K]  ->  dst_p[t][k] = sum_i src[t][i] A_p[k][i]      (u)
//   layout 1: W_p = B_p [K][r_p]  ->  dst_p[t][k] = sum_i src[t][i] B_p[i][k]      (v; n == 1)
// dst_p is fp32 with row stride dst_stride[p].
struct RankJob {
  const uint16_t* src;
  const uint16_t* W[kMaxGroup];
  float* dst[kMaxGroup];
  int32_t r[kMaxGroup];
  int32_t dst_stride[kMaxGroup];
  int32_t n, K, layout, R;
};
struct RankArgs {
  int32_t T;
  int32_t n_jobs;
  RankJob job[kMaxJobs];
};
hipError_t launch_rank_proj(const RankArgs& a, hipStream_t s);

// Gradients reduced over T: for the weights of a job (ranks concatenated in P),
//   G_p = scale_p * sum_t Q[t][c] P[t][off_p + k]
// written [r_p][C] (transpose = 1: dA with Q = x, P = v) or [C][r_p] (transpose = 0: dB
// with Q = dy_p, P = u_p); G_p == null skips that weight.  part: the job's workspace of
// grad_partial_bytes(T, C, R) bytes.  Deterministic: fixed splits, fixed-order sums.
struct GradJob {
  const uint16_t* Q;
  const float* P;
  float* part;
  float* G[kMaxGroup];
  int32_t r[kMaxGroup];
  float scale[kMaxGroup];
  int32_t n, C, R, pstride, transpose;
};
struct GradArgs {
  int32_t T, nsplit, tchunk, accumulate, n_jobs;
  GradJob job[kMaxJobs];
};
size_t grad_partial_bytes(int32_t T, int32_t C, int32_t R);
hipError_t launch_rank_grad(const GradArgs& a, hipStream_t s);

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);

}  // namespace lnf4
