// Fused NF4 (or bf16) frozen-weight GEMMs with the rank-r LoRA epilogue, gfx950 MFMA.
//
// Forward (NT):  y[T, out] = x[T, in] W'^T + s u B^T       M = T, N = out, K = in
// Input grad (NN): dx[T, in] = sum_p dy_p W'_p + s_p v_p A_p   M = T, N = in, K = sum out_p
//
// W' is never materialised: the packed codes are read from the layer buffer and decoded
// in registers (one fp32 product by the block's absmax, one RNE to bf16, exactly as the
// standalone decode does), then fed to v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//
// Tiling.  A workgroup of 4 waves computes a BM x 256 tile (BM = 256 or 128), K-step 64.
// Wave w owns the 64 columns [64w, 64w+64) and all BM rows: BM/32 x 2 MFMA blocks of
// 32x32.  The activation tile (x or dy) is staged through LDS (double buffered, 16-byte
// chunks XOR-swizzled by row).  The K order inside a 64-wide step is permuted so that a
// lane's B fragments for the four 16-wide MFMA steps are 32 consecutive K values: lane
// (n, h) of a 32x32x16 MFMA supplies K = 32h + 8s .. 32h + 8s + 7 at step s.  Both
// operands use the same permutation, so the sum is unchanged.
//
//  * Forward: K runs along a row of W, so each lane loads its own 16 bytes of codes
//    (32 K values of one output column) straight from global memory and decodes them in
//    registers: no LDS round trip for W, and every code is decoded once per workgroup.
//  * dx: K runs across rows of W (W is N-contiguous here), so each thread loads an 8x8
//    sub-block (8 rows x 4 bytes of codes), decodes it, and writes it transposed into LDS
//    (the packed bf16 pairs are formed from two different rows, so the transpose costs
//    nothing beyond the decode).  Waves then read B fragments from LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace lnf4 {

__constant__ float c_gemm_table[16] = LNF4_TABLE_INIT;

constexpr int BN = 256;
constexpr int BK = 64;
constexpr int NTHR = 256;
// largest rank (summed over a group in backward) the fused epilogue stages in LDS
#define LNF4_EPI_RANK 64

__device__ __forceinline__ floatx16 mfma32(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint4 v = make_uint4(a, b, c, d);
  return __builtin_bit_cast(bf16x8, v);
}

// position of 16-byte chunk c of activation-tile row `row` (8 chunks per 128-byte row)
__device__ __forceinline__ int act_pos(int row, int c) { return row * BK + ((c ^ (row & 7)) << 3); }
// position of chunk c of decoded-weight row `n` in the dx kernel's transposed W tile
__device__ __forceinline__ int wt_pos(int n, int c) { return n * BK + ((c ^ ((n ^ (n >> 3)) & 7)) << 3); }

// Field-wise selection of a group member from the kernel arguments with a uniform
// index: every candidate is read with a constant offset and selected in scalar
// registers, so the argument block is never copied to private memory.
#define LNF4_SEL(dst, arr, idx, field)                  \
  do {                                                 \
    dst.field = arr[0].field;                          \
    _Pragma("unroll") for (int q_ = 1; q_ < kMaxGroup; ++q_) \
      if (q_ == (idx)) dst.field = arr[q_].field;      \
  } while (0)

__device__ __forceinline__ FwdProj select_fwd(const FwdArgs& a, int idx) {
  FwdProj P;
  LNF4_SEL(P, a.p, idx, w);
  LNF4_SEL(P, a.p, idx, absmax);
  LNF4_SEL(P, a.p, idx, y);
  LNF4_SEL(P, a.p, idx, u);
  LNF4_SEL(P, a.p, idx, B);
  LNF4_SEL(P, a.p, idx, out_f);
  LNF4_SEL(P, a.p, idx, r);
  LNF4_SEL(P, a.p, idx, scale);
  LNF4_SEL(P, a.p, idx, tile_n0);
  return P;
}

__device__ __forceinline__ DxProj select_dx(const DxArgs& a, int idx) {
  DxProj P;
  LNF4_SEL(P, a.p, idx, w);
  LNF4_SEL(P, a.p, idx, absmax);
  LNF4_SEL(P, a.p, idx, dy);
  LNF4_SEL(P, a.p, idx, v);
  LNF4_SEL(P, a.p, idx, A);
  LNF4_SEL(P, a.p, idx, out_f);
  LNF4_SEL(P, a.p, idx, r);
  LNF4_SEL(P, a.p, idx, scale);
  LNF4_SEL(P, a.p, idx, kb0);
  return P;
}

// =====================================================================================
// Shared epilogue pieces
// =====================================================================================
// Rank-r update folded into the accumulator initialisation.  U [BM][RP] holds the scaled
// rank-r activations (s*u, or s_p*v_p concatenated over a group) split into two bf16
// halves, hi = bf16(U) and lo = bf16(U - hi), so U keeps about 16 significant bits;
// V [256][RP] holds the bf16 adapter rows of the tile's columns (B rows, or A columns).
// acc += hi . V^T + lo . V^T runs on the MFMA units with K = RP (the rank padded to 16
// with zeros), writing straight into the accumulators.
template <int MI>
__device__ __forceinline__ void rank_update(floatx16 (&acc)[MI][2], const uint16_t* Uh, const uint16_t* Ul,
                                            const uint16_t* V, int RP, int l32, int h, int nc0, int nc1) {
  for (int ks = 0; ks < RP; ks += 16) {
    const bf16x8 b0 = *(const bf16x8*)&V[nc0 * RP + ks + 8 * h];
    const bf16x8 b1 = *(const bf16x8*)&V[nc1 * RP + ks + 8 * h];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = 32 * i + l32;
      const bf16x8 ah = *(const bf16x8*)&Uh[row * RP + ks + 8 * h];
      const bf16x8 al = *(const bf16x8*)&Ul[row * RP + ks + 8 * h];
      acc[i][0] = mfma32(ah, b0, acc[i][0]);
      acc[i][1] = mfma32(ah, b1, acc[i][1]);
      acc[i][0] = mfma32(al, b0, acc[i][0]);
      acc[i][1] = mfma32(al, b1, acc[i][1]);
    }
  }
}

__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  const __bf16 h = (__bf16)v;
  const __bf16 l = (__bf16)(v - (float)h);
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, l);
}

template <int BM>
constexpr int epi_bytes() { return (2 * BM + BN) * LNF4_EPI_RANK * 2; }

// =====================================================================================
// Forward
// =====================================================================================
template <int FMT, int BM>
__global__ __launch_bounds__(NTHR, 1) void k_fwd(const FwdArgs args) {
  constexpr int MI = BM / 32;
  constexpr int XL = BM * BK / 8 / NTHR;  // 16-byte chunks per thread per activation tile
  constexpr int XS_BYTES = 2 * BM * BK * 2;
  constexpr int SMEM = XS_BYTES > epi_bytes<BM>() ? XS_BYTES : epi_bytes<BM>();
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ float lut[16];
  uint16_t* xs0 = (uint16_t*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  if (tid < 16) lut[tid] = c_gemm_table[tid];

  const int nb = args.n_tiles_m * args.n_tiles_n;
  const int tile = xcd_remap(blockIdx.x, nb);
  const int tm = tile % args.n_tiles_m, tn = tile / args.n_tiles_m;
  int pi = 0;
#pragma unroll
  for (int q = 1; q < kMaxGroup; ++q)
    if (q < args.n_proj && tn >= args.p[q].tile_n0) pi = q;
  const FwdProj P = select_fwd(args, pi);

  const int M = args.M, K = args.K, out_f = P.out_f;
  const int m0 = tm * BM;
  const int nloc0 = (tn - P.tile_n0) * BN;
  const int nk = K / BK;

  // B-operand rows: columns n = nloc0 + 64*wave + 32*j + l32 (clamped; results discarded)
  const uint8_t* wrow[2];
  const float* arow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int n = nloc0 + 64 * wave + 32 * j + l32;
    n = n < out_f ? n : out_f - 1;
    if (FMT == 0) {
      wrow[j] = (const uint8_t*)P.w + (size_t)n * (K / 2) + 16 * h;
      arow[j] = P.absmax + (size_t)n * (K / 64);
    } else {
      wrow[j] = (const uint8_t*)P.w + (size_t)n * K * 2 + 64 * h;
      arow[j] = nullptr;
    }
  }
  // activation tile rows (clamped; rows >= M only feed discarded outputs)
  const int xc = tid & 7;
  const uint16_t* xbase = args.x + (size_t)m0 * K;
  uint32_t xoff[XL];
#pragma unroll
  for (int q = 0; q < XL; ++q) {
    const int rr = q * 32 + (tid >> 3);
    const int lr = (m0 + rr < M) ? rr : (M - 1 - m0);
    xoff[q] = (uint32_t)lr * (uint32_t)K + (uint32_t)(xc * 8);
  }

  constexpr int WL = (FMT == 0) ? 1 : 4;  // 16-byte loads per B column per K-step
  u32x4 xr[XL];
  u32x4 wr[2][WL];
  float ar[2] = {0.f, 0.f};

  // ---- accumulators start at the rank-r LoRA term s * u[m, :] . B[n, :]
  const int nc0 = 64 * wave + l32, nc1 = nc0 + 32;
  floatx16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  if (P.u != nullptr && P.r > 0) {
    const int r = P.r, RP = (r + 15) & ~15;
    uint16_t* Uh = (uint16_t*)smem;
    uint16_t* Ul = Uh + BM * RP;
    uint16_t* V = Ul + BM * RP;
    for (int idx = tid; idx < BM * RP; idx += NTHR) {
      const int mm = idx / RP, kk = idx - mm * RP, gm = m0 + mm;
      const float uv = (gm < M && kk < r) ? P.scale * P.u[(size_t)gm * r + kk] : 0.0f;
      split_bf16(uv, Uh[idx], Ul[idx]);
    }
    for (int idx = tid; idx < BN * RP; idx += NTHR) {
      const int nn = idx / RP, kk = idx - nn * RP, n = nloc0 + nn;
      V[idx] = (n < out_f && kk < r) ? P.B[(size_t)n * r + kk] : (uint16_t)0;
    }
    __syncthreads();
    rank_update<MI>(acc, Uh, Ul, V, RP, l32, h, nc0, nc1);
    __syncthreads();
  }

#define LNF4_LOAD_X(kb_)                                                         \
  _Pragma("unroll") for (int q = 0; q < XL; ++q) xr[q] = *(const u32x4*)(xbase + xoff[q] + (kb_)*BK);
#define LNF4_STORE_X(buf_)                                                       \
  _Pragma("unroll") for (int q = 0; q < XL; ++q)                                   \
    *(u32x4*)&xs0[(buf_)*BM * BK + act_pos(q * 32 + (tid >> 3), xc)] = xr[q];
#define LNF4_LOAD_W(kb_, dst, adst)                                              \
  _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                  \
    if (FMT == 0) {                                                              \
      dst[j][0] = *(const u32x4*)(wrow[j] + (kb_) * (BK / 2));                   \
      adst[j] = arow[j][(kb_)];                                                  \
    } else {                                                                     \
      _Pragma("unroll") for (int s = 0; s < 4; ++s)                              \
        dst[j][s] = *(const u32x4*)(wrow[j] + (kb_) * BK * 2 + 16 * s);          \
      adst[j] = 0.f;                                                             \
    }                                                                            \
  }

  LNF4_LOAD_X(0);
  LNF4_LOAD_W(0, wr, ar);
  LNF4_STORE_X(0);
  __syncthreads();

  for (int kb = 0; kb < nk; ++kb) {
    const int cur = kb & 1;
    // Prefetch the next K-block (the last iteration re-reads its own block: no branch,
    // so the loads stay ahead of the MFMA work instead of being merged with the stores).
    const int kn = kb + 1 < nk ? kb + 1 : kb;
    u32x4 wn[2][WL];
    float an[2];
    LNF4_LOAD_X(kn);
    LNF4_LOAD_W(kn, wn, an);
    const uint16_t* xt = xs0 + cur * BM * BK;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 b0, b1;
      if (FMT == 0) {
        const uint32_t c0 = wr[0][0][s];
        const uint32_t c1 = wr[1][0][s];
        uint32_t o[4];
        decode8(c0, ar[0], lut, o);
        b0 = as_bf16x8(o[0], o[1], o[2], o[3]);
        decode8(c1, ar[1], lut, o);
        b1 = as_bf16x8(o[0], o[1], o[2], o[3]);
      } else {
        b0 = __builtin_bit_cast(bf16x8, wr[0][s]);
        b1 = __builtin_bit_cast(bf16x8, wr[1][s]);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const bf16x8 a = *(const bf16x8*)&xt[act_pos(32 * i + l32, 4 * h + s)];
        acc[i][0] = mfma32(a, b0, acc[i][0]);
        acc[i][1] = mfma32(a, b1, acc[i][1]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // the other buffer was last read before the previous barrier: safe to overwrite
    LNF4_STORE_X(cur ^ 1);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int s = 0; s < WL; ++s) wr[j][s] = wn[j][s];
      ar[j] = an[j];
    }
    __syncthreads();
  }

#undef LNF4_LOAD_X
#undef LNF4_STORE_X
#undef LNF4_LOAD_W
  // ---- store bf16
  const int n0g = nloc0 + nc0, n1g = nloc0 + nc1;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    __builtin_amdgcn_sched_barrier(0);  // bound the accumulator reads that are live at once
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);
      const int gm = m0 + row;
      if (gm >= M) continue;
      const float v0 = acc[i][0][q], v1 = acc[i][1][q];
      uint16_t* yr = P.y + (size_t)gm * out_f;
      if (n0g < out_f) yr[n0g] = __builtin_bit_cast(uint16_t, (__bf16)v0);
      if (n1g < out_f) yr[n1g] = __builtin_bit_cast(uint16_t, (__bf16)v1);
    }
  }
}

// =====================================================================================
// Input gradient
// =====================================================================================
template <int FMT, int BM>
__global__ __launch_bounds__(NTHR, 1) void k_dx(const DxArgs args) {
  constexpr int MI = BM / 32;
  constexpr int AL = BM * BK / 8 / NTHR;
  constexpr int MAIN_BYTES = 2 * BM * BK * 2 + 2 * BN * BK * 2;
  constexpr int SMEM = MAIN_BYTES > epi_bytes<BM>() ? MAIN_BYTES : epi_bytes<BM>();
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ float lut[16];
  uint16_t* as0 = (uint16_t*)smem;            // [2][BM*BK] activation (dy) tiles
  uint16_t* ws0 = as0 + 2 * BM * BK;          // [2][BN*BK] decoded, transposed W tiles

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  if (tid < 16) lut[tid] = c_gemm_table[tid];

  const int nb = args.n_tiles_m * args.n_tiles_n;
  const int tile = xcd_remap(blockIdx.x, nb);
  const int tm = tile % args.n_tiles_m, tn = tile / args.n_tiles_m;
  const int M = args.M, N = args.N;
  const int m0 = tm * BM, n0 = tn * BN;

  // activation (dy) tile loader mapping
  const int ac = tid & 7;
  int arow_[AL];
#pragma unroll
  for (int q = 0; q < AL; ++q) {
    const int gm = m0 + q * 32 + (tid >> 3);
    arow_[q] = gm < M ? gm : M - 1;
  }
  // weight sub-block loader mapping: rows k0 + 8*kb8 + i, columns n0 + 8*nb8 + e
  const int kb8 = tid >> 5, nb8 = tid & 31;
  const int ncol = n0 + 8 * nb8;
  const bool col_ok = ncol < N;

  // projection of a K-block (uniform)
  auto proj_of = [&](int kb) {
    int pi = 0;
#pragma unroll
    for (int q = 1; q < kMaxGroup; ++q)
      if (q < args.n_proj && kb >= args.p[q].kb0) pi = q;
    return pi;
  };

  u32x4 ar[AL];
  uint32_t wraw[8][FMT == 0 ? 1 : 4];
  float wa[8];

  // prefetch K-block kb_ of the group: dy chunk (16 B per thread per 32 rows) and an 8x8
  // sub-block of W (8 rows x 4 bytes of codes, or 8 rows x 16 bytes of bf16)
#define LNF4_DX_LOAD(kb_)                                                                      \
  {                                                                                            \
    const DxProj P = select_dx(args, proj_of(kb_));                                            \
    const int k0 = ((kb_) - P.kb0) * BK;                                                       \
    const int Kp = P.out_f;                                                                    \
    const int kk = k0 + 8 * ac;                                                                \
    const bool aok = kk < Kp;                                                                  \
    const int kkc = aok ? kk : 0; /* always a valid address; the value is masked */           \
    _Pragma("unroll") for (int q = 0; q < AL; ++q) {                                           \
      const u32x4 v_ = *(const u32x4*)(P.dy + (size_t)arow_[q] * Kp + kkc);                    \
      ar[q] = aok ? v_ : u32x4{0, 0, 0, 0};                                                    \
    }                                                                                          \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                            \
      const int k = k0 + 8 * kb8 + i;                                                          \
      const bool ok = col_ok && k < Kp;                                                        \
      const int kc = ok ? k : 0, cc = col_ok ? ncol : 0;                                       \
      if (FMT == 0) {                                                                          \
        const uint32_t c_ = *(const uint32_t*)((const uint8_t*)P.w + (size_t)kc * (N / 2) + cc / 2); \
        const float a_ = P.absmax[(size_t)kc * (N / 64) + cc / 64];                            \
        wraw[i][0] = ok ? c_ : 0x77777777u; /* code 7 is the zero level */                    \
        wa[i] = ok ? a_ : 0.0f;                                                                \
      } else {                                                                                 \
        const u32x4 v_ = *(const u32x4*)((const uint16_t*)P.w + (size_t)kc * N + cc);          \
        wraw[i][0] = ok ? v_.x : 0u;                                                           \
        wraw[i][FMT == 0 ? 0 : 1] = ok ? v_.y : 0u;                                            \
        wraw[i][FMT == 0 ? 0 : 2] = ok ? v_.z : 0u;                                            \
        wraw[i][FMT == 0 ? 0 : 3] = ok ? v_.w : 0u;                                            \
      }                                                                                        \
    }                                                                                          \
  }
  // store the prefetched dy chunk, and decode + transpose the W sub-block into LDS:
  // column e of the sub-block holds element e of each of the 8 rows (element 2b is the
  // high nibble of byte b); pairs of consecutive rows pack into one dword
#define LNF4_DX_STORE(buf_)                                                                    \
  {                                                                                            \
    uint16_t* at_ = as0 + (buf_) * BM * BK;                                                    \
    uint16_t* wt_ = ws0 + (buf_) * BN * BK;                                                    \
    _Pragma("unroll") for (int q = 0; q < AL; ++q)                                             \
      *(u32x4*)&at_[act_pos(q * 32 + (tid >> 3), ac)] = ar[q];                                 \
    _Pragma("unroll") for (int e = 0; e < 8; ++e) {                                            \
      u32x4 o;                                                                                 \
      if (FMT == 0) {                                                                          \
        const int sh = 8 * (e >> 1) + ((e & 1) ? 0 : 4);                                       \
        float f[8];                                                                            \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) f[i] = lut[(wraw[i][0] >> sh) & 15u] * wa[i]; \
        o.x = pack_bf16x2(f[0], f[1]);                                                         \
        o.y = pack_bf16x2(f[2], f[3]);                                                         \
        o.z = pack_bf16x2(f[4], f[5]);                                                         \
        o.w = pack_bf16x2(f[6], f[7]);                                                         \
      } else {                                                                                 \
        const int wd = e >> 1, sh = (e & 1) * 16;                                              \
        uint32_t hv[8];                                                                        \
        _Pragma("unroll") for (int i = 0; i < 8; ++i) hv[i] = (wraw[i][FMT == 0 ? 0 : wd] >> sh) & 0xffffu; \
        o.x = hv[0] | (hv[1] << 16);                                                           \
        o.y = hv[2] | (hv[3] << 16);                                                           \
        o.z = hv[4] | (hv[5] << 16);                                                           \
        o.w = hv[6] | (hv[7] << 16);                                                           \
      }                                                                                        \
      *(u32x4*)&wt_[wt_pos(8 * nb8 + e, kb8)] = o;                                             \
    }                                                                                          \
  }

  // ---- accumulators start at the rank-R LoRA term: the ranks of every adapted projection
  // concatenated, each projection's v pre-scaled by its s:
  //   U[row][off+k] = s_p v_p[row][k],   V[col][off+k] = A_p[k][col]
  const int nc0 = 64 * wave + l32, nc1 = nc0 + 32;
  floatx16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  int R = 0;
  for (int pi = 0; pi < args.n_proj; ++pi) {
    const DxProj P = select_dx(args, pi);
    if (P.v != nullptr && P.r > 0) R += P.r;
  }
  if (R > 0) {
    const int RP = (R + 15) & ~15;
    uint16_t* Uh = (uint16_t*)smem;
    uint16_t* Ul = Uh + BM * RP;
    uint16_t* V = Ul + BM * RP;
    for (int idx = tid; idx < BM * RP; idx += NTHR) Uh[idx] = Ul[idx] = 0;
    for (int idx = tid; idx < BN * RP; idx += NTHR) V[idx] = 0;
    __syncthreads();
    int off = 0;
    for (int pi = 0; pi < args.n_proj; ++pi) {
      const DxProj P = select_dx(args, pi);
      if (P.v == nullptr || P.r <= 0) continue;
      const int r = P.r;
      for (int idx = tid; idx < BM * r; idx += NTHR) {
        const int mm = idx / r, kk = idx - mm * r, gm = m0 + mm;
        if (gm < M) split_bf16(P.scale * P.v[(size_t)gm * r + kk], Uh[mm * RP + off + kk], Ul[mm * RP + off + kk]);
      }
      for (int idx = tid; idx < BN * r; idx += NTHR) {
        const int kk = idx / BN, nn = idx - kk * BN, n = n0 + nn;
        if (n < N) V[nn * RP + off + kk] = P.A[(size_t)kk * N + n];
      }
      off += r;
    }
    __syncthreads();
    rank_update<MI>(acc, Uh, Ul, V, RP, l32, h, nc0, nc1);
  }

  __syncthreads();  // lut ready; LoRA staging no longer read
  LNF4_DX_LOAD(0);
  LNF4_DX_STORE(0);
  __syncthreads();

  const int nkb = args.total_kb;
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    LNF4_DX_LOAD(kb + 1 < nkb ? kb + 1 : kb);  // unconditional prefetch (see k_fwd)
    const uint16_t* at = as0 + cur * BM * BK;
    const uint16_t* wt = ws0 + cur * BN * BK;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 b0 = *(const bf16x8*)&wt[wt_pos(64 * wave + l32, 4 * h + s)];
      const bf16x8 b1 = *(const bf16x8*)&wt[wt_pos(64 * wave + 32 + l32, 4 * h + s)];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const bf16x8 a = *(const bf16x8*)&at[act_pos(32 * i + l32, 4 * h + s)];
        acc[i][0] = mfma32(a, b0, acc[i][0]);
        acc[i][1] = mfma32(a, b1, acc[i][1]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    LNF4_DX_STORE(cur ^ 1);
    __syncthreads();
  }

#undef LNF4_DX_LOAD
#undef LNF4_DX_STORE
  // ---- store bf16 (optionally accumulating into the existing dx)
  const int n0g = n0 + nc0, n1g = n0 + nc1;
  const bool c0ok = n0g < N, c1ok = n1g < N;
  if (args.accumulate) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int gm = m0 + 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);
        uint16_t* dr = args.dx + (size_t)gm * N;
        if (gm < M && c0ok) dr[n0g] = __builtin_bit_cast(uint16_t, (__bf16)(acc[i][0][q] + bf16_to_f32(dr[n0g])));
        if (gm < M && c1ok) dr[n1g] = __builtin_bit_cast(uint16_t, (__bf16)(acc[i][1][q] + bf16_to_f32(dr[n1g])));
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int gm = m0 + 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);
        uint16_t* dr = args.dx + (size_t)gm * N;
        if (gm < M && c0ok) dr[n0g] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][0][q]);
        if (gm < M && c1ok) dr[n1g] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][1][q]);
      }
    }
  }
}

// =====================================================================================
// Launchers
// =====================================================================================
static int pick_bm(int M, int tiles_n_256) {
  // 256-row tiles decode each weight element once per 256 rows; fall back to 128 rows
  // when 256-row tiles would leave most of the 256 compute units idle.
  const int t256 = ((M + 255) / 256) * tiles_n_256;
  if (t256 >= 192 || M <= 128) return t256 >= 192 ? 256 : 128;
  return 128;
}

hipError_t launch_fwd(const FwdArgs& a0, int fmt, hipStream_t s) {
  FwdArgs a = a0;
  if (a.M <= 0 || a.n_tiles_n <= 0) return hipSuccess;
  const int bm = pick_bm(a.M, a.n_tiles_n);
  a.n_tiles_m = (a.M + bm - 1) / bm;
  const dim3 grid(a.n_tiles_m * a.n_tiles_n), block(NTHR);
  if (fmt == 0) {
    if (bm == 256) hipLaunchKernelGGL((k_fwd<0, 256>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_fwd<0, 128>), grid, block, 0, s, a);
  } else {
    if (bm == 256) hipLaunchKernelGGL((k_fwd<1, 256>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_fwd<1, 128>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_dx(const DxArgs& a0, int fmt, hipStream_t s) {
  DxArgs a = a0;
  if (a.M <= 0 || a.N <= 0 || a.total_kb <= 0) return hipSuccess;
  a.n_tiles_n = (a.N + BN - 1) / BN;
  const int bm = pick_bm(a.M, a.n_tiles_n);
  a.n_tiles_m = (a.M + bm - 1) / bm;
  const dim3 grid(a.n_tiles_m * a.n_tiles_n), block(NTHR);
  if (fmt == 0) {
    if (bm == 256) hipLaunchKernelGGL((k_dx<0, 256>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_dx<0, 128>), grid, block, 0, s, a);
  } else {
    if (bm == 256) hipLaunchKernelGGL((k_dx<1, 256>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_dx<1, 128>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace lnf4
