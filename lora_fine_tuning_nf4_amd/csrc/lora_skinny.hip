// Skinny rank-r LoRA products with wavefront-level reductions (no padded MFMA tiles).
//
//   u  = x  A^T   [T, r]   (forward; also the recompute when u was not saved)
//   v  = dy B     [T, r]   (first step of the backward)
//   dA = s v^T x  [r, in]  (reduction over T)
//   dB = s dy^T u [out, r] (reduction over T)
//
// u and v (k_rank_proj; from 16 concatenated ranks on, k_rank_tile below): one launch
// serves several jobs (blockIdx.y).  A job is one
// activation matrix src [T, K] and the weights that multiply it; weights that share src
// (q and v both read x) are one job with their ranks concatenated (R = sum r_p <= 64), so
// src is read from HBM once.  A workgroup owns RB rows of src and all of K: its waves (as
// many as K/8 needs lanes, 1 to 8) take interleaved K slices (lane = 8 consecutive K, one
// 16-byte load), each lane accumulates RB x RMAX partial dot products, a butterfly
// reduce-scatter across the wave leaves each lane NV/64 finished slice totals, and the
// waves' totals are added in a fixed order through LDS.  Results are fp32 and
// deterministic.
//
// dA and dB (k_rank_grad): a job is Q [T, C] bf16 times P [T, R] fp32 reduced over T, for
// the weights whose ranks are concatenated in P (dA of every adapted projection of a
// group shares Q = x; each dB has its own Q = dy_p).  Each lane owns CPL columns and all
// R ranks; P rows are the same for every lane of a wave and are read as LDS broadcasts from
// a per-wave staging slice, 16 rows at a time.  The 4 waves of a workgroup split the
// workgroup's T range and add through LDS in a fixed order; workgroups along T write
// partials that k_rank_grad_reduce adds in a fixed order (no atomics).
#include "common.hpp"
#include "kernels.hpp"

namespace lnf4 {

// Butterfly reduce-scatter of NV (64 or 128) per-lane values over the 64 lanes of a wave:
// at each xor step a lane keeps one half of its values and adds the partner's copy of
// that half, so NV values need NV/2 + NV/4 + ... + NV/64 shuffles.  On return
// v[j] (j < NV/64) is the wave total of value index lane * (NV/64) + j.
template <int NV>
__device__ __forceinline__ void wave_reduce_scatter(float (&v)[NV], int lane) {
  static_assert(NV == 64 || NV == 128, "NV");  // one or two finished values per lane
#pragma unroll
  for (int st = 0; st < 6; ++st) {  // a counted loop, so it unrolls and v stays in registers
    const int mask = 32 >> st, w = NV >> (st + 1);
    const uint32_t m = (lane & mask) != 0 ? 0xffffffffu : 0u;
#pragma unroll
    for (int i = 0; i < w; ++i) {
      // choose by bit masks: a select between two array elements would be folded into a
      // lane-dependent index, which sends the whole array to scratch memory
      const uint32_t a = __float_as_uint(v[i]), b = __float_as_uint(v[i + w]);
      const float send = __uint_as_float((a & m) | (b & ~m));
      const float keep = __uint_as_float((b & m) | (a & ~m));
      v[i] = keep + __shfl_xor(send, mask, 64);
    }
  }
}

// projection that owns concatenated rank kk (ranks r[0], r[1], ... laid end to end);
// off = its first concatenated rank
__device__ __forceinline__ int rank_owner(const int32_t* r, int n, int kk, int& off) {
  int p = 0;
  off = 0;
  while (p + 1 < n && kk >= off + r[p]) {
    off += r[p];
    ++p;
  }
  return p;
}

__device__ __forceinline__ void unpack8(const u32x4& q, float f[8]) {
  f[0] = bf16_lo(q[0]); f[1] = bf16_hi(q[0]);
  f[2] = bf16_lo(q[1]); f[3] = bf16_hi(q[1]);
  f[4] = bf16_lo(q[2]); f[5] = bf16_hi(q[2]);
  f[6] = bf16_lo(q[3]); f[7] = bf16_hi(q[3]);
}

// ==================================================================== u = x A^T, v = dy B
// RMAX: rank capacity of the job (R <= RMAX); RB rows of src per workgroup.
template <int RMAX>
struct RankCfg {
  static constexpr int RB = 64 / RMAX;
  static constexpr int NV = RB * RMAX;  // per-lane accumulators
};

template <int RMAX, int LAYOUT>
__global__ __launch_bounds__(512) void k_rank_proj(const RankArgs args) {
  constexpr int RB = RankCfg<RMAX>::RB, NV = RankCfg<RMAX>::NV;
  __shared__ float part[8][NV];
  __shared__ const uint16_t* wrow[RMAX];   // layout 0: row pointer of each concatenated rank
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = blockDim.x >> 6;  // waves of this launch (1..8)
  const RankJob& J = args.job[blockIdx.y];
  const int T = args.T, K = J.K, R = J.R, n = J.n;
  const int t0 = blockIdx.x * RB;
  if (t0 >= T) return;  // whole workgroup
  if (LAYOUT == 0 && tid < RMAX) {
    int off;
    const int p = rank_owner(J.r, n, tid, off);
    wrow[tid] = (tid < R) ? J.W[p] + (size_t)(tid - off) * K : nullptr;
  }
  __syncthreads();

  float acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.f;
  const int nch = K / 8;
  for (int c = 64 * wave + lane; c - lane < nch; c += 64 * nw) {  // wave-uniform trip count
    const bool ok = c < nch;
    const int cc = ok ? c : 0;
    u32x4 xq[RB];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const int t = (t0 + rr < T) ? t0 + rr : T - 1;
      xq[rr] = *(const u32x4*)(J.src + (size_t)t * K + 8 * cc);
      if (!ok) xq[rr] = u32x4{0, 0, 0, 0};
    }
    if (LAYOUT == 0) {
      float xf[RB][8];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) unpack8(xq[rr], xf[rr]);
#pragma unroll
      for (int k = 0; k < RMAX; ++k) {
        if (k < R) {
          float wf[8];
          unpack8(*(const u32x4*)(wrow[k] + 8 * cc), wf);
#pragma unroll
          for (int rr = 0; rr < RB; ++rr) {
            float s = acc[rr * RMAX + k];
#pragma unroll
            for (int e = 0; e < 8; ++e) s += xf[rr][e] * wf[e];
            acc[rr * RMAX + k] = s;
          }
        }
      }
    } else {
      // B [K][r]: the lane's 8 rows are 8r contiguous bf16 (16r bytes); eight ranks of one
      // row at a time
      const uint16_t* bp = J.W[0] + (size_t)(8 * cc) * R;
      const bool vec = R == RMAX && ((uintptr_t)J.W[0] & 15) == 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int k8 = 0; k8 < RMAX / 8; ++k8) {
          if (8 * k8 < R) {
            if (RMAX >= 32) __builtin_amdgcn_sched_barrier(0);  // bound the B rows in flight
            float wf[8];
            if (vec) {
              unpack8(*(const u32x4*)(bp + e * RMAX + 8 * k8), wf);
            } else {
#pragma unroll
              for (int j = 0; j < 8; ++j) wf[j] = (8 * k8 + j < R) ? bf16_to_f32(bp[e * R + 8 * k8 + j]) : 0.f;
            }
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) {
              const uint32_t wd = xq[rr][e >> 1];
              const float xe = (e & 1) ? bf16_hi(wd) : bf16_lo(wd);
#pragma unroll
              for (int j = 0; j < 8; ++j) acc[rr * RMAX + 8 * k8 + j] += xe * wf[j];
            }
          }
        }
      }
    }
  }
  wave_reduce_scatter<NV>(acc, lane);
#pragma unroll
  for (int j = 0; j < NV / 64; ++j) part[wave][lane * (NV / 64) + j] = acc[j];
  __syncthreads();
  if (tid < NV) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < nw; ++w) s += part[w][tid];
    const int rr = tid / RMAX, kk = tid % RMAX, t = t0 + rr;
    if (kk < R && t < T) {
      int off;
      const int p = rank_owner(J.r, n, kk, off);
      J.dst[p][(size_t)t * J.dst_stride[p] + (kk - off)] = s;
    }
  }
}

// ---------------------------------------------------------------- tiled u / v (LDS-staged)
// The same products with the weights staged in LDS and reused across rows: a workgroup owns
// 8 rows of src and all ranks of its job and walks K in chunks; the chunk of src and the
// chunk of the job's weights (transposed to [rank][K] for layout 1) are staged in LDS as
// fp32, and each lane accumulates an OT x OK block of (row, rank) dot products over its
// wave's quarter of the chunk with 16-byte LDS reads.  The four waves' partial sums are
// added in a fixed order at the end.  The next chunk's loads are in flight while the
// current chunk is multiplied.
template <int RMAX>
struct TileCfg {
  static constexpr int OK = RMAX >= 16 ? 2 : 1;    // ranks per lane
  static constexpr int KP = RMAX / OK;             // lanes along ranks
  static constexpr int TP = 64 / KP;               // lanes along rows
  static constexpr int OT = 8 / TP;                // rows per lane
  static constexpr int TB = 8;                     // rows per workgroup
  static constexpr int KC = 8192 / RMAX;           // K per chunk (32 KB of fp32 weights)
  static constexpr int STR = KC + 4;               // LDS row stride (floats): rows start 16 B apart in the banks
  static constexpr int AL = RMAX * KC / 8 / 256;   // layout 0: 16-byte weight loads per thread and chunk
  static constexpr int XL = (TB * KC / 8 + 255) / 256;  // 16-byte src loads per thread and chunk
  static constexpr int BL = RMAX * KC / 256;       // layout 1: weight elements per thread and chunk
};

template <int RMAX, int LAYOUT>
__global__ __launch_bounds__(256) void k_rank_tile(const RankArgs args) {
  using C = TileCfg<RMAX>;
  constexpr int OT = C::OT, OK = C::OK, TB = C::TB, KC = C::KC, STR = C::STR;
  static_assert(C::TP * OT == TB && C::KP * OK == RMAX, "lane layout");
  __shared__ __attribute__((aligned(16))) float ws_[RMAX * STR];   // weights [rank][K chunk]
  __shared__ __attribute__((aligned(16))) float xs_[TB * STR];     // src rows [row][K chunk]
  __shared__ const uint16_t* wrow[RMAX];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const RankJob& J = args.job[blockIdx.y];
  const int T = args.T, K = J.K, R = J.R, n = J.n;
  const int t0 = blockIdx.x * TB;
  if (t0 >= T) return;  // whole workgroup
  if (LAYOUT == 0 && tid < RMAX) {
    int off;
    const int p = rank_owner(J.r, n, tid, off);
    wrow[tid] = (tid < R) ? J.W[p] + (size_t)(tid - off) * K : nullptr;
  }
  // ranks past R stay zero in every chunk
  for (int e = tid; e < (RMAX - R) * STR; e += 256) ws_[R * STR + e] = 0.f;
  __syncthreads();

  // ---- chunk loads into registers (zeros past K or T)
  u32x4 xr[C::XL];
  u32x4 ar[LAYOUT == 0 ? C::AL : 1];
  uint32_t br[LAYOUT == 1 ? C::BL : 1];
  u32x4 bv[LAYOUT == 1 ? C::BL / 8 : 1];
  // layout 1 with whole 16-byte pieces of B rows (R a multiple of 8, B 16-byte aligned)
  const bool bvec = LAYOUT == 1 && (R & 7) == 0 && (((uintptr_t)J.W[0]) & 15) == 0;
  auto load = [&](int kc) {
#pragma unroll
    for (int q = 0; q < C::XL; ++q) {
      const int e = 256 * q + tid, row = e / (KC / 8), c8 = e % (KC / 8);
      const int t = t0 + row < T ? t0 + row : T - 1, i = kc + 8 * c8;
      xr[q] = (row < TB && i < K) ? *(const u32x4*)(J.src + (size_t)t * K + i) : u32x4{0u, 0u, 0u, 0u};
    }
    if (LAYOUT == 0) {
#pragma unroll
      for (int q = 0; q < C::AL; ++q) {
        const int e = 256 * q + tid, k = e / (KC / 8), c8 = e % (KC / 8), i = kc + 8 * c8;
        ar[q] = (k < R && i < K) ? *(const u32x4*)(wrow[k] + i) : u32x4{0u, 0u, 0u, 0u};
      }
    } else if (bvec) {
      // B [K][R] row-major, 16-byte rows pieces: 8 ranks of one K row per load
#pragma unroll
      for (int q = 0; q < C::BL / 8; ++q) {
        const int e = 256 * q + tid, i = e / (RMAX / 8), k8 = 8 * (e % (RMAX / 8));
        bv[q] = (k8 < R && kc + i < K) ? *(const u32x4*)(J.W[0] + (size_t)(kc + i) * R + k8) : u32x4{0u, 0u, 0u, 0u};
      }
    } else {
      // B [K][R] row-major: consecutive threads read consecutive elements
#pragma unroll
      for (int q = 0; q < C::BL; ++q) {
        const int e = 256 * q + tid, i = e / RMAX, k = e % RMAX;
        br[q] = (k < R && kc + i < K) ? (uint32_t)J.W[0][(size_t)(kc + i) * R + k] : 0u;
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int q = 0; q < C::XL; ++q) {
      const int e = 256 * q + tid, row = e / (KC / 8), c8 = e % (KC / 8);
      if (row < TB) {
        float f[8];
        unpack8(xr[q], f);
        *(float4*)&xs_[row * STR + 8 * c8] = make_float4(f[0], f[1], f[2], f[3]);
        *(float4*)&xs_[row * STR + 8 * c8 + 4] = make_float4(f[4], f[5], f[6], f[7]);
      }
    }
    if (LAYOUT == 0) {
#pragma unroll
      for (int q = 0; q < C::AL; ++q) {
        const int e = 256 * q + tid, k = e / (KC / 8), c8 = e % (KC / 8);
        if (k < R) {
          float f[8];
          unpack8(ar[q], f);
          *(float4*)&ws_[k * STR + 8 * c8] = make_float4(f[0], f[1], f[2], f[3]);
          *(float4*)&ws_[k * STR + 8 * c8 + 4] = make_float4(f[4], f[5], f[6], f[7]);
        }
      }
    } else if (bvec) {
#pragma unroll
      for (int q = 0; q < C::BL / 8; ++q) {
        const int e = 256 * q + tid, i = e / (RMAX / 8), k8 = 8 * (e % (RMAX / 8));
        if (k8 < R) {
          float f[8];
          unpack8(bv[q], f);
#pragma unroll
          for (int j = 0; j < 8; ++j) ws_[(k8 + j) * STR + i] = f[j];
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < C::BL; ++q) {
        const int e = 256 * q + tid, i = e / RMAX, k = e % RMAX;
        if (k < R) ws_[k * STR + i] = bf16_to_f32((uint16_t)br[q]);
      }
    }
  };

  const int tp = lane / C::KP, kp = lane % C::KP;
  float acc[OT][OK];
#pragma unroll
  for (int a = 0; a < OT; ++a)
#pragma unroll
    for (int b = 0; b < OK; ++b) acc[a][b] = 0.f;
  const int nchunk = (K + KC - 1) / KC;
  load(0);
  for (int c = 0; c < nchunk; ++c) {
    __syncthreads();  // every wave is done with the previous chunk
    store();
    __syncthreads();
    if (c + 1 < nchunk) load((c + 1) * KC);
    // this wave's quarter of the chunk, 4 K per step
#pragma unroll 4
    for (int i = wave * (KC / 4); i < (wave + 1) * (KC / 4); i += 4) {
      float4 xv[OT], wv[OK];
#pragma unroll
      for (int a = 0; a < OT; ++a) xv[a] = *(const float4*)&xs_[(tp * OT + a) * STR + i];
#pragma unroll
      for (int b = 0; b < OK; ++b) wv[b] = *(const float4*)&ws_[(kp * OK + b) * STR + i];
#pragma unroll
      for (int a = 0; a < OT; ++a)
#pragma unroll
        for (int b = 0; b < OK; ++b) {
          float s_ = acc[a][b];
          s_ += xv[a].x * wv[b].x;
          s_ += xv[a].y * wv[b].y;
          s_ += xv[a].z * wv[b].z;
          s_ += xv[a].w * wv[b].w;
          acc[a][b] = s_;
        }
    }
  }
  // fixed-order sum of the four waves' partials
  __syncthreads();
  float* red = ws_;  // [4 waves][64 lanes][OT*OK]
#pragma unroll
  for (int a = 0; a < OT; ++a)
#pragma unroll
    for (int b = 0; b < OK; ++b) red[(wave * 64 + lane) * (OT * OK) + a * OK + b] = acc[a][b];
  __syncthreads();
  for (int o = tid; o < 64 * OT * OK; o += 256) {
    const float s_ = red[o] + red[64 * OT * OK + o] + red[2 * 64 * OT * OK + o] + red[3 * 64 * OT * OK + o];
    const int l = o / (OT * OK), a = (o % (OT * OK)) / OK, b = o % OK;
    const int t = t0 + (l / C::KP) * OT + a, kk = (l % C::KP) * OK + b;
    if (t < T && kk < R) {
      int off;
      const int p = rank_owner(J.r, n, kk, off);
      J.dst[p][(size_t)t * J.dst_stride[p] + (kk - off)] = s_;
    }
  }
}

// ==================================================================== dA, dB partials
template <int RMAX>
struct GradCfg {
  static constexpr int CPL = RMAX <= 32 ? 2 : 1;  // columns per lane
  static constexpr int COLS = 64 * CPL;          // columns per workgroup
};

// XOR swizzle of a lane's NVAL wave sums in LDS: the lanes' rows start NVAL floats apart,
// so without it the 64 lanes of one store instruction hit only 64/NVAL of the 64 banks
template <int NVAL>
__device__ __forceinline__ int red_swz(int l) { return (NVAL >= 64 ? l : l / (64 / NVAL)) & (NVAL - 1); }

template <int RMAX>
__global__ __launch_bounds__(256) void k_rank_grad(const GradArgs args) {
  constexpr int CPL = GradCfg<RMAX>::CPL, COLS = GradCfg<RMAX>::COLS;
  constexpr int NVAL = CPL * RMAX;
  constexpr int RU = 16;  // rows per group
  __shared__ float red[4][64 * NVAL];
  __shared__ __attribute__((aligned(16))) float pst[4][RU][RMAX];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const GradJob& J = args.job[blockIdx.z];
  const int T = args.T, C = J.C, R = J.R;
  const int cb = blockIdx.x * COLS;
  if (cb >= C) return;  // whole workgroup (jobs have different widths)
  const int split = blockIdx.y;
  const int tb = split * args.tchunk;
  const int te = tb + args.tchunk < T ? tb + args.tchunk : T;
  // this wave's rows: a quarter of the workgroup's range
  const int q4 = (te - tb + 3) / 4;
  const int wb = tb + wave * q4;
  const int we = wb + q4 < te ? wb + q4 : te;
  const int c0 = cb + lane * CPL;
  const bool ok = c0 < C;  // C is even when CPL == 2
  const int cc = ok ? c0 : 0;

  float acc[CPL][RMAX];
#pragma unroll
  for (int e = 0; e < CPL; ++e)
#pragma unroll
    for (int k = 0; k < RMAX; ++k) acc[e][k] = 0.f;
  // The wave's rows in groups of RU.  The group's P rows are staged in the wave's own LDS
  // slice (zero past R and past the wave's last row), so the products read them without
  // per-rank bounds branches.  The next group's P and Q loads are issued before the
  // current group's products, so their latency hides behind them.  Products run in row
  // order: every sum is the same sequence of adds.
  static_assert(RU * RMAX % 64 == 0, "staging covers whole waves");
  constexpr int PL = RU * RMAX / 64;  // staged P values per lane per group
  float* pw = &pst[wave][0][0];
  float pn[PL], qn[RU][CPL];
#define LNF4_RG_LOAD(t_)                                                                 \
  {                                                                                      \
    _Pragma("unroll") for (int j = 0; j < PL; ++j) {                                     \
      const int i = 64 * j + lane, u = i / RMAX, k = i % RMAX;                           \
      pn[j] = (k < R && (t_) + u < we) ? J.P[(size_t)((t_) + u) * J.pstride + k] : 0.f;  \
    }                                                                                    \
    _Pragma("unroll") for (int u = 0; u < RU; ++u) {                                     \
      const int tr = (t_) + u < we ? (t_) + u : we - 1; /* past the end: P is zero */   \
      if (CPL == 2) {                                                                    \
        const uint32_t w = *(const uint32_t*)(J.Q + (size_t)tr * C + cc);                \
        qn[u][0] = bf16_lo(w);                                                           \
        qn[u][CPL - 1] = bf16_hi(w);                                                     \
      } else {                                                                           \
        qn[u][0] = bf16_to_f32(J.Q[(size_t)tr * C + cc]);                                \
      }                                                                                  \
    }                                                                                    \
  }
  if (wb < we) LNF4_RG_LOAD(wb);
  for (int t = wb; t < we; t += RU) {
    float q[RU][CPL];
#pragma unroll
    for (int u = 0; u < RU; ++u)
#pragma unroll
      for (int e = 0; e < CPL; ++e) q[u][e] = qn[u][e];
    __builtin_amdgcn_wave_barrier();  // the previous group's reads of the slice come first
#pragma unroll
    for (int j = 0; j < PL; ++j) pw[64 * j + lane] = pn[j];
    if (t + RU < we) LNF4_RG_LOAD(t + RU);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int u = 0; u < RU; ++u) {
#pragma unroll
      for (int k4 = 0; k4 < RMAX; k4 += 4) {
        const floatx4 p4 = *(const floatx4*)&pw[u * RMAX + k4];  // same address in every lane
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int e = 0; e < CPL; ++e) acc[e][k4 + kk] += p4[kk] * q[u][e];
      }
    }
  }
#undef LNF4_RG_LOAD
#pragma unroll
  for (int e = 0; e < CPL; ++e)
#pragma unroll
    for (int k = 0; k < RMAX; ++k) red[wave][lane * NVAL + ((e * RMAX + k) ^ red_swz<NVAL>(lane))] = acc[e][k];
  __syncthreads();
  // fixed-order sum of the 4 waves; partial layout [split][c][R]
  float* dst = J.part + (size_t)split * C * R;
  for (int i = tid; i < 64 * NVAL; i += 256) {
    const int l = i / NVAL, e = (i % NVAL) / RMAX, k = i % RMAX, ri = l * NVAL + ((i % NVAL) ^ red_swz<NVAL>(l));
    const float s = red[0][ri] + red[1][ri] + red[2][ri] + red[3][ri];
    const int c = cb + l * CPL + e;
    if (c < C && k < R) dst[(size_t)c * R + k] = s;
  }
}

// G_p = s_p * sum over splits, written [r_p][C] (transpose) or [C][r_p]; one thread per
// (job, c, k) of the concatenated ranks
__global__ __launch_bounds__(256) void k_rank_grad_reduce(const GradArgs args) {
  const GradJob& J = args.job[blockIdx.y];
  const int64_t n = (int64_t)J.C * J.R;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  float s = 0.f;
  for (int sp = 0; sp < args.nsplit; ++sp) s += J.part[(size_t)sp * n + idx];
  const int c = (int)(idx / J.R), kk = (int)(idx % J.R);
  int off;
  const int p = rank_owner(J.r, J.n, kk, off);
  float* G = J.G[p];
  if (G == nullptr) return;  // this weight's gradient was not asked for
  const int k = kk - off, r = J.r[p];
  s *= J.scale[p];
  const size_t o = J.transpose ? (size_t)k * J.C + c : (size_t)c * r + k;
  G[o] = args.accumulate ? G[o] + s : s;
}

__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// ==================================================================== launchers
static int rank_cap(int R) { return R <= 8 ? 8 : R <= 16 ? 16 : R <= 32 ? 32 : 64; }

// Zero-fill with a kernel rather than a memset node, so the call is safe to capture.
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

template <int LAYOUT>
static hipError_t launch_rank_tile(const RankArgs& a, int rmax, hipStream_t s) {
  const dim3 grid((a.T + 7) / 8, a.n_jobs), blk(256);
  switch (rmax) {
    case 8: hipLaunchKernelGGL((k_rank_tile<8, LAYOUT>), grid, blk, 0, s, a); break;
    case 16: hipLaunchKernelGGL((k_rank_tile<16, LAYOUT>), grid, blk, 0, s, a); break;
    case 32: hipLaunchKernelGGL((k_rank_tile<32, LAYOUT>), grid, blk, 0, s, a); break;
    default: hipLaunchKernelGGL((k_rank_tile<64, LAYOUT>), grid, blk, 0, s, a); break;
  }
  return hipGetLastError();
}

template <int LAYOUT>
static hipError_t launch_rank_layout(const RankArgs& a, int rmax, hipStream_t s) {
  // staged weights pay off from 16 concatenated ranks on; with 8 ranks the per-row kernel
  // below is faster (8B shapes: v of q and v in 17 us against 23 us; u of q|v, 16 ranks, in
  // 24.6 us against 25.2 us, and 12-17 us against 19-40 us for the 0.5B shapes' 16-64)
  if (rmax >= 16) return launch_rank_tile<LAYOUT>(a, rmax, s);
  // one lane per 8 K of the widest job, 1 to 8 waves: small K does not leave most lanes idle
  int kmax = 8;
  for (int j = 0; j < a.n_jobs; ++j) kmax = a.job[j].K > kmax ? a.job[j].K : kmax;
  const int waves = (kmax / 8 + 63) / 64;
  const dim3 blk(64 * (waves < 1 ? 1 : (waves > 8 ? 8 : waves)));
  switch (rmax) {
    case 8:
      hipLaunchKernelGGL((k_rank_proj<8, LAYOUT>), dim3((a.T + RankCfg<8>::RB - 1) / RankCfg<8>::RB, a.n_jobs), blk,
                         0, s, a);
      break;
    case 16:
      hipLaunchKernelGGL((k_rank_proj<16, LAYOUT>), dim3((a.T + RankCfg<16>::RB - 1) / RankCfg<16>::RB, a.n_jobs),
                         blk, 0, s, a);
      break;
    case 32:
      hipLaunchKernelGGL((k_rank_proj<32, LAYOUT>), dim3((a.T + RankCfg<32>::RB - 1) / RankCfg<32>::RB, a.n_jobs),
                         blk, 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((k_rank_proj<64, LAYOUT>), dim3((a.T + RankCfg<64>::RB - 1) / RankCfg<64>::RB, a.n_jobs),
                         blk, 0, s, a);
      break;
  }
  return hipGetLastError();
}

// every job of one launch must have the same layout
hipError_t launch_rank_proj(const RankArgs& a, hipStream_t s) {
  if (a.T <= 0 || a.n_jobs <= 0) return hipSuccess;
  int rmax = 8;
  for (int j = 0; j < a.n_jobs; ++j) rmax = rank_cap(a.job[j].R) > rmax ? rank_cap(a.job[j].R) : rmax;
  return a.job[0].layout == 0 ? launch_rank_layout<0>(a, rmax, s) : launch_rank_layout<1>(a, rmax, s);
}

// most T splits a launch may use (at least 64 rows each, at most 32 splits): the partial
// workspace of a job is sized for this many
static int grad_max_split(int T) {
  const int ns = T / 64;
  return ns < 1 ? 1 : (ns > 32 ? 32 : ns);
}

size_t grad_partial_bytes(int32_t T, int32_t C, int32_t R) {
  if (T <= 0 || R <= 0 || C <= 0) return 0;
  return (size_t)grad_max_split(T) * (size_t)C * (size_t)R * sizeof(float);
}

hipError_t launch_rank_grad(const GradArgs& a0, hipStream_t s) {
  if (a0.T <= 0 || a0.n_jobs <= 0) return hipSuccess;
  GradArgs a = a0;
  int rmax = 8, cmax = 0;
  int64_t nmax = 0;
  for (int j = 0; j < a.n_jobs; ++j) {
    rmax = rank_cap(a.job[j].R) > rmax ? rank_cap(a.job[j].R) : rmax;
    cmax = a.job[j].C > cmax ? a.job[j].C : cmax;
    const int64_t n = (int64_t)a.job[j].C * a.job[j].R;
    nmax = n > nmax ? n : nmax;
  }
  // T splits: enough workgroups with work (about 576, a little over two per compute unit)
  // for narrow jobs, at least 8 splits when T allows; the split count depends only on the
  // shapes, so results stay deterministic
  const int cols = rmax <= 32 ? GradCfg<8>::COLS : GradCfg<64>::COLS;
  int cb_total = 0;
  for (int j = 0; j < a.n_jobs; ++j) cb_total += (a.job[j].C + cols - 1) / cols;
  const int maxs = grad_max_split(a.T), mins = maxs < 8 ? maxs : 8;
  int ns = (576 + cb_total - 1) / (cb_total > 0 ? cb_total : 1);
  a.nsplit = ns < mins ? mins : (ns > maxs ? maxs : ns);
  a.tchunk = (a.T + a.nsplit - 1) / a.nsplit;
  const dim3 blk(256);
  switch (rmax) {
    case 8:
      hipLaunchKernelGGL(k_rank_grad<8>, dim3((cmax + GradCfg<8>::COLS - 1) / GradCfg<8>::COLS, a.nsplit, a.n_jobs),
                         blk, 0, s, a);
      break;
    case 16:
      hipLaunchKernelGGL(k_rank_grad<16>, dim3((cmax + GradCfg<16>::COLS - 1) / GradCfg<16>::COLS, a.nsplit, a.n_jobs),
                         blk, 0, s, a);
      break;
    case 32:
      hipLaunchKernelGGL(k_rank_grad<32>, dim3((cmax + GradCfg<32>::COLS - 1) / GradCfg<32>::COLS, a.nsplit, a.n_jobs),
                         blk, 0, s, a);
      break;
    default:
      hipLaunchKernelGGL(k_rank_grad<64>, dim3((cmax + GradCfg<64>::COLS - 1) / GradCfg<64>::COLS, a.nsplit, a.n_jobs),
                         blk, 0, s, a);
      break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_rank_grad_reduce, dim3((unsigned)((nmax + 255) / 256), a.n_jobs), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lnf4
