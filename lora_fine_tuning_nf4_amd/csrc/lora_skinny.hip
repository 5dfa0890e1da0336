// Skinny rank-r LoRA products on the matrix cores (v_mfma_f32_16x16x32_bf16).
//
//   u  = x  A^T   [T, r]   (forward; also the recompute when u was not saved)
//   v  = dy B     [T, r]   (first step of the backward)
//   dA = s v^T x  [r, in]  (reduction over T)
//   dB = s dy^T u [out, r] (reduction over T)
//
// These are dense contractions whose arithmetic intensity is the rank: with the ranks of a
// group concatenated (up to 64) an fp32 multiply-add per product would bound them on the
// vector ALU well below the HBM rate, so they run as bf16 MFMAs with fp32 accumulation.
// For u and v both operands are bf16 already and every product is exact in fp32.  For dA
// and dB the fp32 operand (v or u) is split into bf16 hi + lo halves (16 bits of its
// mantissa kept; two MFMAs per tile).
//
// MFMA operand layout used throughout: lane l holds row (l & 15) of the A operand and
// column (l & 15) of the B operand, each with 8 contraction indices chosen by l >> 4; lane
// l receives column (l & 15), rows 4 (l >> 4) + 0..3 of the 16 x 16 result.  Which 8
// indices a lane group holds is free as long as A and B agree lane by lane.
//
// u and v (k_lora_proj): one launch serves several jobs (blockIdx.y).  A job is one
// activation matrix src [T, K] and the weights that multiply it; weights that share src
// (q and v both read x) are one job with their ranks concatenated (R = sum r_p <= 64), so
// src is read from HBM once.  dA and dB (k_lora_grad): a job is Q [T, C] bf16 reduced
// against P [T, R] fp32 over T; T splits write partials that k_rank_grad_reduce adds in a
// fixed order.  Every sum runs in an order fixed by the shapes alone: results are
// deterministic.
#include "common.hpp"
#include "kernels.hpp"

namespace lnf4 {

typedef short v4s_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16): in each group of 16 lanes, lane a + 4c gives
// the address of the 4-element run (columns 4a .. 4a+3) of row c of a row-major 4 x 16
// block, and lane i receives column i of the four rows, in row order.
__device__ __forceinline__ v4s_t lds_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)p);
}

__device__ __forceinline__ bf16x8 join8(const v4s_t& lo, const v4s_t& hi) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
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

// ==================================================================== u = x A^T, v = dy B
// Pointer to the row of concatenated rank kk in the matrix of the projection that owns it
// (row length ld).  Every projection's pointer and rank are read with a constant index
// (scalar loads of the kernel arguments) and the lane's one is chosen by compares; ranks
// past the job's read the first projection's first row.
__device__ __forceinline__ const uint16_t* rank_row(const RankJob& J, int kk, int64_t ld) {
  const uint16_t* w = J.W[0];
  int off = 0;
#pragma unroll
  for (int p = 0; p < kMaxGroup; ++p) {
    if (p < J.n) {
      const int r = J.r[p];
      if (kk >= off && kk < off + r) w = J.W[p] + (size_t)(kk - off) * ld;
      off += r;
    }
  }
  return w;
}

// A workgroup owns BT (16, or 8 when 16-row workgroups would leave compute units idle)
// rows of src and every rank of its job (RT tiles of 16); with 8 rows the MFMA's other 8
// A rows read zeros.  Its 8 waves
// take the job's K in super-steps of 64 (wave w: steps w, w + 8, ...).  Half h of a
// super-step (K 32h .. 32h+31) feeds one MFMA; lane l reads the 8 K at 8 (l >> 4) of it
// from its row, so one load instruction reads 64 contiguous bytes of each of 16 rows.
// src is read through a buffer resource: a step past K reads zeros without touching
// memory.  Weights in layout 0 (A [r][K], K contiguous) load straight into the B operand
// the same way (a step past K re-reads the last one; never used).  In layout 1 (B [K][r],
// r contiguous) each wave copies the 64 weight rows of its super-step into its own LDS
// slice (row-major, ranks padded to RT * 16 with zeros) and reads them back transposed.
// PD super-steps are in flight per wave in a register ring; the steady-state block has no
// branches, so the compiler's wait before a step's MFMAs leaves the later steps' loads
// outstanding.  The waves' partial sums add through LDS in wave order; the K split
// depends on K alone, so a result does not depend on the other ranks of its job or on PD.
template <int RT, int LAYOUT, int PD_, int BT = 16>
__global__ __launch_bounds__(512) void k_lora_proj(const RankArgs args) {
  // register budget: 8 steps in flight for the 1-2 tile shapes, at most 2 for the widest
  constexpr int PD = (LAYOUT == 1 && RT == 4 && PD_ > 2) ? 2 : ((RT > 2 || (LAYOUT == 1 && RT > 1)) && PD_ > 4 ? 4 : PD_);
  constexpr int NW = 8, BTM = 16, R16 = 16 * RT;  // BTM: rows of the MFMA tile
  static_assert(BT == 16 || BT == 8, "workgroup rows");
  constexpr int SL = LAYOUT == 1 ? 64 * R16 : 8;  // staging slice per wave (bf16 elements)
  constexpr int PL = 2 * RT;                       // layout 1: 16-byte weight pieces per lane
  constexpr uint32_t OOB = 0x80000000u;            // buffer offset past any resource
  __shared__ float red[NW * BTM * R16];
  __shared__ __attribute__((aligned(16))) uint16_t bst[NW * SL];
  const RankJob& J = args.job[blockIdx.y];
  const int T = args.T, K = J.K, R = J.R;
  const int t0 = blockIdx.x * BT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int nss = (K + 63) >> 6;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // A operand: row t0 + l16 (rows past T repeat row T - 1; their sums are not stored;
  // lanes past the workgroup's BT rows read zeros)
  const rsrc_t srs = make_rsrc(J.src, (int64_t)T * K * 2);
  const int trow = t0 + l16 < T ? t0 + l16 : T - 1;
  const bool arow = l16 < BT;
  const uint32_t aoff = 2u * ((uint32_t)trow * (uint32_t)K + 8u * g);
  // layout 0: weight row of concatenated rank 16 rt + l16
  const uint16_t* wrow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) wrow[rt] = LAYOUT == 0 ? rank_row(J, 16 * rt + l16, K) + 8 * g : J.W[0];
  // layout 1: one projection, r = R; 16-byte pieces when r % 8 == 0 and B is 16-byte
  // aligned, single elements otherwise
  const uint16_t* Bw = J.W[0];
  const bool vec = LAYOUT == 1 && R % 8 == 0 && ((uintptr_t)Bw & 15) == 0;
  const rsrc_t brs = make_rsrc(Bw, (int64_t)K * R * 2);
  const int rp = R >= 8 ? R / 8 : 1;  // pieces per weight row (vec)
  uint16_t* slice = bst + wave * SL;
  if (LAYOUT == 1) {
    // zero the slice once: the staged rows only overwrite ranks < r
#pragma unroll
    for (int i = 0; i < SL / 512; ++i) *(u32x4*)(slice + 8 * (lane + 64 * i)) = zero;
  }

  floatx4 acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = floatx4{0.f, 0.f, 0.f, 0.f};

  struct Frag {
    u32x4 a[2];
    u32x4 b[LAYOUT == 0 ? RT : 1][2];
    u32x4 w[LAYOUT == 1 ? PL : 1];
  };
  const auto load = [&](Frag& f, int s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = 64 * s + 32 * h + 8 * g;  // K % 8 == 0: a half is all in or all out
      f.a[h] = LNF4_BUF_LD128(srs, (k < K && arow) ? aoff + 128u * s + 64u * h : OOB, 0);
      if (LAYOUT == 0) {
        const int kc = (k < K ? 64 * s + 32 * h : K - 8 - 8 * g);  // clamped into the row
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) f.b[rt][h] = *(const u32x4*)(wrow[rt] + kc);
      }
    }
    if (LAYOUT == 1 && vec) {
      // piece e = lane + 64 q of the 64 x r block: row e / rp, ranks 8 (e % rp) .. +7;
      // rows past K read zeros
#pragma unroll
      for (int q = 0; q < PL; ++q) {
        const int e = lane + 64 * q, kr = e / rp;
        const uint32_t off = 2u * ((uint32_t)(64 * s + kr) * (uint32_t)R + 8u * (uint32_t)(e - kr * rp));
        f.w[q] = LNF4_BUF_LD128(brs, q < rp ? off : OOB, 0);
      }
    }
  };
  const auto compute = [&](const Frag& f, int s) {
    bf16x8 bop[RT][2];
    if (LAYOUT == 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int h = 0; h < 2; ++h) bop[rt][h] = __builtin_bit_cast(bf16x8, f.b[rt][h]);
    } else {
      __builtin_amdgcn_wave_barrier();  // the previous super-step's reads of the slice come first
      if (vec) {
#pragma unroll
        for (int q = 0; q < PL; ++q) {
          if (q < rp) {
            const int e = lane + 64 * q, kr = e / rp;
            *(u32x4*)(slice + kr * R16 + 8 * (e - kr * rp)) = f.w[q];
          }
        }
      } else {
        const int kb = 64 * s;
        for (int e = lane; e < 64 * R; e += 64) {
          const int kr = e / R, c = e - kr * R;
          slice[kr * R16 + c] = kb + kr < K ? Bw[(size_t)(kb + kr) * R + c] : (uint16_t)0;
        }
      }
      __builtin_amdgcn_wave_barrier();
      const int rr = 8 * g + (l16 >> 2), cc = 4 * (l16 & 3);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint16_t* p = slice + (rr + 32 * h) * R16 + 16 * rt + cc;
          bop[rt][h] = join8(lds_tr16(p), lds_tr16(p + 4 * R16));
        }
    }
    // src halves past K are zeros (buffer bounds), which also cancels the re-read weights
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        if (16 * rt < R) acc[rt] = mfma16(__builtin_bit_cast(bf16x8, f.a[h]), bop[rt][h], acc[rt]);
  };

  // register ring: slot i holds step base + NW i
  Frag f[PD];
#pragma unroll
  for (int i = 0; i < PD; ++i) load(f[i], wave + NW * i);
  int base = wave;
  // steady state: every slot computes its step and refills with a real one
  for (; base + NW * (2 * PD - 1) < nss; base += NW * PD) {
#pragma unroll
    for (int i = 0; i < PD; ++i) {
      compute(f[i], base + NW * i);
      load(f[i], base + NW * (PD + i));
    }
  }
  // drain: at most 2 PD - 1 steps remain; the first PD are in the ring
#pragma unroll
  for (int i = 0; i < PD; ++i) {
    const int st = base + NW * i;
    if (st < nss) {
      compute(f[i], st);
      if (st + NW * PD < nss) load(f[i], st + NW * PD);
    }
  }
#pragma unroll
  for (int i = 0; i < PD; ++i) {
    const int st = base + NW * (PD + i);
    if (st < nss) compute(f[i], st);
  }

  // fixed-order sum of the 8 waves' partials
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * BTM + 4 * g + i) * R16 + 16 * rt + l16] = acc[rt][i];
  __syncthreads();
  for (int idx = tid; idx < BT * R; idx += 64 * NW) {
    const int row = idx / R, kk = idx - row * R, t = t0 + row;
    if (t >= T) continue;
    float sum = red[row * R16 + kk];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum += red[(w * BTM + row) * R16 + kk];
    float* d = J.dst[0];
    int off = 0;
#pragma unroll
    for (int p = 0; p < kMaxGroup; ++p) {
      if (p < J.n) {
        const int r = J.r[p];
        if (kk >= off && kk < off + r) d = J.dst[p] + (size_t)t * J.dst_stride[p] + (kk - off);
        off += r;
      }
    }
    *d = sum;
  }
}

// ==================================================================== dA = s v^T x, dB = s dy^T u
// A workgroup (4 waves) owns 64 columns of Q and the T range of its split, in steps of 32
// rows.  Each step stages Q [32][64] bf16 (16-byte chunks swizzled by row so that a
// transposing read touches every bank pair once) and P [32][R] split into bf16 hi and lo
// halves in LDS, double-buffered, the loads of the step after next in flight meanwhile.
// Wave w multiplies the transpose of its 16 columns of Q (A operand: 16 columns x 32 rows)
// by the transposed halves of P (B operand, per rank tile): 2 MFMAs per tile and step.
// Waves own disjoint columns, so a split's partial needs no reduction inside the
// workgroup; it is written [split][C][R].
__device__ __forceinline__ int grad_swz(int row) { return 2 * ((row >> 3) & 3); }

template <int RT>
__global__ __launch_bounds__(256) void k_lora_grad(const GradArgs args) {
  constexpr int R16 = 16 * RT;
  constexpr int QS = 32 * 64, PS = 32 * R16;  // bf16 elements per stage
  constexpr int PQ = (8 * R16 + 255) / 256;   // 4-element P pieces per thread and step
  constexpr uint32_t OOB = 0x80000000u;       // buffer offset past any resource
  __shared__ __attribute__((aligned(16))) uint16_t qs[2][QS];
  __shared__ __attribute__((aligned(16))) uint16_t ph[2][PS];
  __shared__ __attribute__((aligned(16))) uint16_t pl[2][PS];
  const GradJob& J = args.job[blockIdx.z];
  const int T = args.T, C = J.C, R = J.R;
  const int cb = blockIdx.x * 64;
  if (cb >= C) return;  // whole workgroup (jobs have different widths)
  const int split = blockIdx.y;
  const int tb = split * args.tchunk;
  const int te = tb + args.tchunk < T ? tb + args.tchunk : T;
  const int nsteps = te > tb ? (te - tb + 31) / 32 : 0;  // an empty split writes zeros
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;

  // staging roles: Q chunk (row tq, 8 columns at 8 cq); P pieces (row, 4 ranks).  Loads go
  // through buffer resources: rows past the split, columns past C and ranks past R read
  // zeros without touching memory, so every load is issued unconditionally.
  const rsrc_t qrs = make_rsrc(J.Q, (int64_t)T * C * 2);
  const rsrc_t prs = make_rsrc(J.P, (int64_t)T * J.pstride * 4);
  const int tq = tid >> 3, cq = tid & 7;
  const bool cq_ok = cb + 8 * cq < C;  // C % 8 == 0: a chunk is all in or all out
  const int qdst = tq * 64 + 8 * (cq ^ grad_swz(tq));
  struct Set {
    u32x4 q;
    float p[PQ][4];
  };
  const auto load = [&](Set& S, int st) {
    const int t = tb + 32 * st + tq;
    S.q = LNF4_BUF_LD128(qrs, (cq_ok && t < te) ? 2u * ((uint32_t)t * (uint32_t)C + (uint32_t)(cb + 8 * cq)) : OOB, 0);
    // P ranks past R read whatever follows (they only reach result columns that are
    // never stored); rows past the split read zeros
#pragma unroll
    for (int q = 0; q < PQ; ++q) {
      const int e = tid + 256 * q, row = e / (R16 / 4), k0 = 4 * (e - row * (R16 / 4));
      const int tp = tb + 32 * st + row;
      const uint32_t off = (e < 8 * R16 && tp < te) ? 4u * ((uint32_t)tp * (uint32_t)J.pstride + (uint32_t)k0) : OOB;
#pragma unroll
      for (int j = 0; j < 4; ++j) S.p[q][j] = __uint_as_float(LNF4_BUF_LD32(prs, off, 4 * j));
    }
  };
  const auto store = [&](const Set& S, int buf) {
    *(u32x4*)&qs[buf][qdst] = S.q;
#pragma unroll
    for (int q = 0; q < PQ; ++q) {
      const int e = tid + 256 * q, row = e / (R16 / 4), k0 = 4 * (e - row * (R16 / 4));
      if (e < 8 * R16) {
        uint32_t hw[2], lw[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float a = S.p[q][2 * j], b = S.p[q][2 * j + 1];
          hw[j] = pack_bf16x2(a, b);
          lw[j] = pack_bf16x2(a - bf16_lo(hw[j]), b - bf16_hi(hw[j]));
        }
        *(uint2*)&ph[buf][row * R16 + k0] = make_uint2(hw[0], hw[1]);
        *(uint2*)&pl[buf][row * R16 + k0] = make_uint2(lw[0], lw[1]);
      }
    }
  };

  floatx4 acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
  // operand reads: lane group g takes rows 8g .. 8g+7 of the step (two 4-row reads)
  const int rr = 8 * g + (l16 >> 2);
  const int qc = 16 * wave + 4 * (l16 & 3);
  const int qa0 = rr * 64 + 8 * ((qc >> 3) ^ grad_swz(rr)) + (qc & 7);
  const int qa1 = (rr + 4) * 64 + 8 * ((qc >> 3) ^ grad_swz(rr + 4)) + (qc & 7);
  const int pa = rr * R16 + 4 * (l16 & 3);
  const auto compute = [&](int buf) {
    const bf16x8 a = join8(lds_tr16(&qs[buf][qa0]), lds_tr16(&qs[buf][qa1]));
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (16 * rt < R) {
        const uint16_t* h0 = &ph[buf][pa + 16 * rt];
        const uint16_t* l0 = &pl[buf][pa + 16 * rt];
        const bf16x8 bh = join8(lds_tr16(h0), lds_tr16(h0 + 4 * R16));
        const bf16x8 bl = join8(lds_tr16(l0), lds_tr16(l0 + 4 * R16));
        acc[rt] = mfma16(a, bh, acc[rt]);
        acc[rt] = mfma16(a, bl, acc[rt]);
      }
    }
  };

  // Step st is staged in LDS buffer st & 1 from register set st & 1; the set of step st + 2
  // is loaded as soon as step st is staged, so two steps' loads are in flight behind the
  // MFMAs.  Steps past the split load and stage zeros that no MFMA reads; loads and stores
  // are unconditional, so the compiler's waits before a store leave the newer set's loads
  // outstanding.
  Set s0, s1;
  load(s0, 0);
  load(s1, 1);
  store(s0, 0);
  load(s0, 2);
  __syncthreads();
  for (int st = 0; st < nsteps; st += 2) {
    compute(0);
    store(s1, 1);
    load(s1, st + 3);
    __syncthreads();
    if (st + 1 < nsteps) compute(1);
    store(s0, 0);
    load(s0, st + 4);
    __syncthreads();
  }

  // partial of this split: column cb + 16 wave + 4g + i, rank 16 rt + l16
  float* dst = J.part + (size_t)split * C * R;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int k = 16 * rt + l16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = cb + 16 * wave + 4 * g + i;
      if (c < C && k < R) dst[(size_t)c * R + k] = acc[rt][i];
    }
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
// Zero-fill with a kernel rather than a memset node, so the call is safe to capture.
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

template <int LAYOUT, int PD, int BT>
static void launch_proj_bt(const RankArgs& a, int rt, hipStream_t s) {
  const dim3 grid((a.T + BT - 1) / BT, a.n_jobs), blk(512);
  switch (rt) {
    case 1: hipLaunchKernelGGL((k_lora_proj<1, LAYOUT, PD, BT>), grid, blk, 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_lora_proj<2, LAYOUT, PD, BT>), grid, blk, 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_lora_proj<3, LAYOUT, PD, BT>), grid, blk, 0, s, a); break;
    default: hipLaunchKernelGGL((k_lora_proj<4, LAYOUT, PD, BT>), grid, blk, 0, s, a); break;
  }
}

static int proj_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    hipDeviceProp_t prop;
    cus = (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess &&
           prop.multiProcessorCount > 0) ? prop.multiProcessorCount : 256;
  }
  return cus;
}

template <int LAYOUT, int PD>
static void launch_proj_pd(const RankArgs& a, int rt, hipStream_t s) {
  // 8-row workgroups when 16-row ones would fill under one round of the compute units:
  // the launch reads src at the rate of the units it runs on (Llama-8B u of q|v at
  // T = 2048: 128 workgroups of 16 rows)
  if ((int64_t)((a.T + 15) / 16) * a.n_jobs < proj_cus()) launch_proj_bt<LAYOUT, PD, 8>(a, rt, s);
  else launch_proj_bt<LAYOUT, PD, 16>(a, rt, s);
}

template <int LAYOUT>
static void launch_proj_layout(const RankArgs& a, int rt, int spw, hipStream_t s) {
  // ring depth: the steps of the wave with the most (1, 2, 4 or 8; the kernel caps it by
  // its register budget)
  if (spw <= 1) launch_proj_pd<LAYOUT, 1>(a, rt, s);
  else if (spw <= 3) launch_proj_pd<LAYOUT, 2>(a, rt, s);
  else if (spw <= 7) launch_proj_pd<LAYOUT, 4>(a, rt, s);
  else launch_proj_pd<LAYOUT, 8>(a, rt, s);
}

// every job of one launch must have the same layout
hipError_t launch_rank_proj(const RankArgs& a, hipStream_t s) {
  if (a.T <= 0 || a.n_jobs <= 0) return hipSuccess;
  int rmax = 1, kmax = 8;
  for (int j = 0; j < a.n_jobs; ++j) {
    if (a.job[j].R > 64 || a.job[j].K % 8 != 0 || a.job[j].K < 8) return hipErrorInvalidValue;  // tile and load contract
    if ((int64_t)a.T * a.job[j].K * 2 > 0x7fffffff) return hipErrorInvalidValue;                 // 32-bit buffer offsets
    rmax = a.job[j].R > rmax ? a.job[j].R : rmax;
    kmax = a.job[j].K > kmax ? a.job[j].K : kmax;
  }
  const int rt = (rmax + 15) / 16;
  const int spw = ((kmax + 63) / 64 + 7) / 8;  // super-steps of the busiest wave
  if (a.job[0].layout == 0) launch_proj_layout<0>(a, rt, spw, s);
  else launch_proj_layout<1>(a, rt, spw, s);
  return hipGetLastError();
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
  int rmax = 1, cmax = 0;
  int64_t nmax = 0;
  for (int j = 0; j < a.n_jobs; ++j) {
    if (a.job[j].R > 64 || a.job[j].C % 8 != 0) return hipErrorInvalidValue;  // tile and load contract
    rmax = a.job[j].R > rmax ? a.job[j].R : rmax;
    cmax = a.job[j].C > cmax ? a.job[j].C : cmax;
    const int64_t n = (int64_t)a.job[j].C * a.job[j].R;
    nmax = n > nmax ? n : nmax;
  }
  // T splits: enough workgroups with work (about 576, a little over two per compute unit)
  // for narrow jobs, at least 8 splits when T allows; the split count depends only on the
  // shapes, so results stay deterministic
  int cb_total = 0;
  for (int j = 0; j < a.n_jobs; ++j) cb_total += (a.job[j].C + 63) / 64;
  const int maxs = grad_max_split(a.T), mins = maxs < 8 ? maxs : 8;
  int ns = (576 + cb_total - 1) / (cb_total > 0 ? cb_total : 1);
  a.nsplit = ns < mins ? mins : (ns > maxs ? maxs : ns);
  a.tchunk = (a.T + a.nsplit - 1) / a.nsplit;
  const dim3 grid((cmax + 63) / 64, a.nsplit, a.n_jobs), blk(256);
  switch ((rmax + 15) / 16) {
    case 1: hipLaunchKernelGGL(k_lora_grad<1>, grid, blk, 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_lora_grad<2>, grid, blk, 0, s, a); break;
    case 3: hipLaunchKernelGGL(k_lora_grad<3>, grid, blk, 0, s, a); break;
    default: hipLaunchKernelGGL(k_lora_grad<4>, grid, blk, 0, s, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_rank_grad_reduce, dim3((unsigned)((nmax + 255) / 256), a.n_jobs), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lnf4
