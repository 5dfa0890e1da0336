// Causal grouped-query attention of a decoder layer, forward and backward, on the
// gfx950 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// Layout: q and o are [T, n_heads * D] bf16, k and v [T, n_kv * D]; the T tokens are
// n_seq sequences of seq_len tokens, attention is causal inside each sequence, and query
// head h reads kv head h / (n_heads / n_kv).  Blocks of 64 queries and 64 keys; a
// workgroup is two waves of 32 rows each.
//
// Orientation.  Scores are formed transposed, S^T = K Q^T, so that a lane's accumulator
// column is one query: that query's softmax statistics (running max and sum, its
// log-sum-exp, rowsum(dO o O)) stay in the lane, and the two half-waves that share the
// column combine with one cross-half exchange.  The probabilities then feed the next
// product straight from the accumulators: the 8 values a lane holds for a 16-key step
// are keys {4h..4h+3, 8+4h..8+4h+3} of that step (h = lane / 32), an order the other
// operand (V^T, K^T, Q^T or dO^T) is read in: from a row-major LDS tile with gfx950's
// transposing 16-bit reads.
//
// The probabilities P and the score gradients dS enter their products as a bf16 hi + lo
// pair (two products each), so o, dq, dk and dv carry about 16 significant bits of them
// (a single bf16 would put a 2^-9 relative error on every term, and the gradients of
// tokens attended by many queries sum many terms that cancel).
//
// Backward without atomics (bitwise reproducible): rowsum(dO o O) per query first, then
// dq (a workgroup per query block, looping over its key blocks) and dk, dv (a workgroup
// per key block and query head, looping over the query blocks at or after it; with
// grouped kv heads each writes an fp32 share, and a last pass sums the shares of a kv
// head in head order).
#include <math.h>

#include "common.hpp"
#include "decoder.hpp"

namespace lnf4 {

namespace {

constexpr int BQ = 64;   // queries per staged block (backward dk, dv)
constexpr int BK = 64;   // keys per staged block (forward, backward dq)
// a workgroup is NW waves of 32 rows each (queries in the forward and dq, keys in dk,
// dv): 4 waves share each staged block when the sequence length allows 128-row blocks

__device__ __forceinline__ floatx16 mma(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld16(const uint16_t* p) { return *(const bf16x8*)p; }

// accumulator values 8*hs .. 8*hs+7 (rows 16hs + 8(p>>2) + 4h + (p&3), p = 0..7) as a bf16
// pair hi + lo (lo = bf16(x - hi)): about 16 significant bits through two products, for
// the probabilities and score gradients fed back into MFMAs
__device__ __forceinline__ void rows_bf16_split(const floatx16& c, int hs, bf16x8& hi, bf16x8& lo) {
  uint32_t wh[4], wl[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = c[8 * hs + 2 * j], b = c[8 * hs + 2 * j + 1];
    wh[j] = pack_bf16x2(a, b);
    wl[j] = pack_bf16x2(a - bf16_lo(wh[j]), b - bf16_hi(wh[j]));
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(wh[0], wh[1], wh[2], wh[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(wl[0], wl[1], wl[2], wl[3]));
}

// Row-major [rows][D] bf16 tile whose 16-byte chunks are swizzled by row (chunk c of row r
// at c ^ swz_chunk(r)), for operands read transposed with ds_read_b64_tr_b16: in each
// group of 16 lanes, lane a + 4c names the 4-column run 4a..4a+3 of row c and lane i
// receives column i of those four rows.  A read covers 8 rows and 32 columns; the swizzle
// puts rows r..r+3 on disjoint banks, so it takes the minimum two LDS cycles.
template <int D>
__device__ __forceinline__ int swz_chunk(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }

typedef short v4s_t __attribute__((ext_vector_type(4)));

// A operand of rows m = mbase + l32 of the transpose of a swizzled row-major tile X[r][m],
// for the 16 r of K-step kbase .. kbase+15 in the order rows_bf16_split produces
// (r = kbase + 4h + 0..3, then kbase + 8 + 4h + 0..3)
template <int D>
__device__ __forceinline__ bf16x8 tr16_operand(const uint16_t* X, int mbase, int kbase, int lane) {
  const int h = lane >> 5, c = (lane & 15) >> 2;
  const int col = mbase + 16 * ((lane & 31) >> 4) + 4 * (lane & 3);
  const int r0 = kbase + 4 * h + c, r1 = r0 + 8;
  const uint16_t* p0 = X + r0 * D + 8 * ((col >> 3) ^ swz_chunk<D>(r0)) + (col & 7);
  const uint16_t* p1 = X + r1 * D + 8 * ((col >> 3) ^ swz_chunk<D>(r1)) + (col & 7);
  const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)p0);
  const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)p1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ floatx16 zero16() {
  floatx16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// A 64 x D bf16 block held in registers between its global load and its LDS writes, so
// that the next block's loads are in flight while the current block computes.  Thread
// items are row pairs (2rp, 2rp + 1) x 16-byte chunk c, written either to a padded
// row-major tile (rows read whole) or to a swizzled one (read transposed).
template <int D, int NT>
struct Staged {
  static constexpr int ITEMS = 32 * (D / 8) / NT;
  u32x4 a[ITEMS][2];

  __device__ __forceinline__ void load(const uint16_t* src, int64_t r0, int64_t ld, int64_t c0) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int idx = threadIdx.x + it * NT, rp = idx / (D / 8), c = idx - rp * (D / 8);
      a[it][0] = *(const u32x4*)(src + (r0 + 2 * rp) * ld + c0 + 8 * c);
      a[it][1] = *(const u32x4*)(src + (r0 + 2 * rp + 1) * ld + c0 + 8 * c);
    }
  }
  template <int STRIDE>
  __device__ __forceinline__ void rows(uint16_t* dst) const {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int idx = threadIdx.x + it * NT, rp = idx / (D / 8), c = idx - rp * (D / 8);
      *(u32x4*)&dst[(2 * rp) * STRIDE + 8 * c] = a[it][0];
      *(u32x4*)&dst[(2 * rp + 1) * STRIDE + 8 * c] = a[it][1];
    }
  }
  // row-major, no padding, chunks swizzled for transposing reads (tr16_operand)
  __device__ __forceinline__ void rows_swz(uint16_t* dst) const {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int idx = threadIdx.x + it * NT, rp = idx / (D / 8), c = idx - rp * (D / 8);
      *(u32x4*)&dst[(2 * rp) * D + 8 * (c ^ swz_chunk<D>(2 * rp))] = a[it][0];
      *(u32x4*)&dst[(2 * rp + 1) * D + 8 * (c ^ swz_chunk<D>(2 * rp + 1))] = a[it][1];
    }
  }
};

// accumulator rows d = 32dt + 8j + 4h + 0..3 of column `col` -> out[col][d], scaled, bf16
template <int D>
__device__ __forceinline__ void store_cols(uint16_t* out_row, const floatx16 (&acc)[D / 32], float f, int h) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * dt + 8 * j + 4 * h;
      uint2 w;
      w.x = pack_bf16x2(acc[dt][4 * j + 0] * f, acc[dt][4 * j + 1] * f);
      w.y = pack_bf16x2(acc[dt][4 * j + 2] * f, acc[dt][4 * j + 3] * f);
      *(uint2*)(out_row + d0) = w;
    }
}

}  // namespace

// ------------------------------------------------------------------ forward
// Online softmax over key blocks in base 2: x = s * scale * log2(e), running max m and
// sum l per query, O^T rescaled by 2^(m_old - m_new) when m grows.  lse is stored in
// natural-log units: (m + log2 l) * ln 2.
// Four-wave workgroups are compiled for two workgroups per compute unit (at most 256
// registers per lane), so one workgroup's softmax overlaps the other's MFMAs.
template <int D, int NW>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void k_attn_fwd(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                 const uint16_t* __restrict__ v, int64_t T, int nh, int nkv,
                                                 int64_t S, float sl2e, uint16_t* __restrict__ o,
                                                 float* __restrict__ lse) {
  constexpr int KS = D + 8, NT = 64 * NW, BR = 32 * NW;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BK * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vr[BK * D];  // row-major, swizzled
  const int nqb = (int)(S / BR), n_seq = (int)(T / S);
  const int seq = blockIdx.x % n_seq, qb = nqb - 1 - (int)(blockIdx.x / n_seq);  // longest rows first
  const int hq = blockIdx.y, hk = hq / (nh / nkv);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l32 = lane & 31, h = lane >> 5;
  const int64_t ldq = (int64_t)nh * D, ldk = (int64_t)nkv * D, t0 = (int64_t)seq * S;
  const int qpos = qb * BR + wave * 32 + l32;  // this lane's query, position in its sequence
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int kb_last = (qb * BR + BR - 1) / BK;

  bf16x8 qf[D / 16];
  const uint16_t* qrow = q + (t0 + qpos) * ldq + (int64_t)hq * D;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) qf[s] = ld16(qrow + 16 * s + 8 * h);
  floatx16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = zero16();
  float m = -INFINITY, l = 0.0f;

  Staged<D, NT> pk, pv;
  pk.load(k, t0, ldk, (int64_t)hk * D);
  pv.load(v, t0, ldk, (int64_t)hk * D);
  for (int kb = 0; kb <= kb_last; ++kb) {
    __syncthreads();  // the previous block's LDS reads are done
    pk.template rows<KS>(Ks);
    pv.rows_swz(Vr);
    __syncthreads();
    if (kb < kb_last) {  // the next block's loads fly while this one computes
      pk.load(k, t0 + (int64_t)(kb + 1) * BK, ldk, (int64_t)hk * D);
      pv.load(v, t0 + (int64_t)(kb + 1) * BK, ldk, (int64_t)hk * D);
    }
    floatx16 st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st[t] = zero16();
      bf16x8 kfr[D / 16];
#pragma unroll
      for (int s = 0; s < D / 16; ++s) kfr[s] = ld16(&Ks[(32 * t + l32) * KS + 16 * s + 8 * h]);
      __builtin_amdgcn_sched_barrier(0);  // every fragment read in flight before the products
#pragma unroll
      for (int s = 0; s < D / 16; ++s) st[t] = mma(kfr[s], qf[s], st[t]);
    }
    float bm = -INFINITY;
    // the causal mask only touches the key blocks that reach past this wave's first query
    // (a wave-uniform test); elsewhere every score is kept
    if (kb * BK + BK - 1 > qb * BR + wave_u * 32) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * BK + 32 * t + 8 * (i >> 2) + 4 * h + (i & 3);
          const float x = key > qpos ? -INFINITY : st[t][i] * sl2e;
          st[t][i] = x;
          bm = fmaxf(bm, x);
        }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = st[t][i] * sl2e;
          st[t][i] = x;
          bm = fmaxf(bm, x);
        }
    }
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mn = fmaxf(m, bm);
    // the hardware exponential (v_exp_f32): exp2f adds a rescale for results below 2^-126,
    // which the forward's VALU-bound loop pays for on every element; such probabilities
    // flush to zero here, beside the row maximum's probability 1 they change no sum
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    float rs = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(st[t][i] - mn);
        st[t][i] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 32);
    l = l * alpha + rs;
    m = mn;
    if (__ballot(alpha != 1.0f)) {  // a factor of exactly 1 for every lane changes nothing
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        bf16x8 ph, pl;
        rows_bf16_split(st[t], hs, ph, pl);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const bf16x8 a = tr16_operand<D>(Vr, 32 * dt, 32 * t + 16 * hs, lane);
          oacc[dt] = mma(a, ph, oacc[dt]);
          oacc[dt] = mma(a, pl, oacc[dt]);
        }
      }
  }
  store_cols<D>(o + (t0 + qpos) * ldq + (int64_t)hq * D, oacc, 1.0f / l, h);
  if (h == 0) lse[(int64_t)hq * T + t0 + qpos] = (m + log2f(l)) * 0.69314718055994531f;
}

// ------------------------------------------------------------------ backward
// rowsum(dO o O) per head and token: dsum[h][t]
__global__ __launch_bounds__(256) void k_attn_bwd_dsum(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dO,
                                                       int64_t T, int nh, int D, float* __restrict__ dsum) {
  const int64_t ld = (int64_t)nh * D;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x)
    for (int hh = threadIdx.x; hh < nh; hh += 256) {
      float acc = 0.0f;
      for (int c = 0; c < D / 8; ++c) {
        const u32x4 a = *(const u32x4*)(o + t * ld + (int64_t)hh * D + 8 * c);
        const u32x4 b = *(const u32x4*)(dO + t * ld + (int64_t)hh * D + 8 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc += bf16_lo(a[i]) * bf16_lo(b[i]) + bf16_hi(a[i]) * bf16_hi(b[i]);
      }
      dsum[(int64_t)hh * T + t] = acc;
    }
}

// dq = scale * dS K with dS^T = P^T o (dP^T - dsum), P^T = exp(S^T - lse), dP^T = V dO^T
// two four-wave workgroups per compute unit, as in the forward (dk, dv keep one: their
// accumulators do not fit in 256 registers)
template <int D, int NW>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void k_attn_bwd_dq(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                    const uint16_t* __restrict__ v, const float* __restrict__ lse,
                                                    const uint16_t* __restrict__ dO, const float* __restrict__ dsum,
                                                    int64_t T, int nh, int nkv, int64_t S, float scale, float sl2e,
                                                    uint16_t* __restrict__ dq) {
  constexpr int KS = D + 8, NT = 64 * NW, BR = 32 * NW;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BK * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BK * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Kr[BK * D];  // row-major, swizzled
  const int nqb = (int)(S / BR), n_seq = (int)(T / S);
  const int seq = blockIdx.x % n_seq, qb = nqb - 1 - (int)(blockIdx.x / n_seq);
  const int hq = blockIdx.y, hk = hq / (nh / nkv);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l32 = lane & 31, h = lane >> 5;
  const int64_t ldq = (int64_t)nh * D, ldk = (int64_t)nkv * D, t0 = (int64_t)seq * S;
  const int qpos = qb * BR + wave * 32 + l32;
  const int kb_last = (qb * BR + BR - 1) / BK;

  bf16x8 qf[D / 16], dof[D / 16];
  const int64_t qoff = (t0 + qpos) * ldq + (int64_t)hq * D;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = ld16(q + qoff + 16 * s + 8 * h);
    dof[s] = ld16(dO + qoff + 16 * s + 8 * h);
  }
  const float lse2 = lse[(int64_t)hq * T + t0 + qpos] * 1.44269504088896341f;
  const float dd = dsum[(int64_t)hq * T + t0 + qpos];
  floatx16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = zero16();

  Staged<D, NT> pk, pv;
  pk.load(k, t0, ldk, (int64_t)hk * D);
  pv.load(v, t0, ldk, (int64_t)hk * D);
  for (int kb = 0; kb <= kb_last; ++kb) {
    __syncthreads();
    pk.template rows<KS>(Ks);
    pk.rows_swz(Kr);
    pv.template rows<KS>(Vs);
    __syncthreads();
    if (kb < kb_last) {
      pk.load(k, t0 + (int64_t)(kb + 1) * BK, ldk, (int64_t)hk * D);
      pv.load(v, t0 + (int64_t)(kb + 1) * BK, ldk, (int64_t)hk * D);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      floatx16 st = zero16(), dp = zero16();
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        st = mma(ld16(&Ks[(32 * t + l32) * KS + 16 * s + 8 * h]), qf[s], st);
        dp = mma(ld16(&Vs[(32 * t + l32) * KS + 16 * s + 8 * h]), dof[s], dp);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * BK + 32 * t + 8 * (i >> 2) + 4 * h + (i & 3);
        // masked by a select, not a branch; the hardware exponential, as in the forward
        const float e = __builtin_amdgcn_exp2f(st[i] * sl2e - lse2);
        const float p = key > qpos ? 0.0f : e;
        st[i] = p * (dp[i] - dd);  // dS^T
      }
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        bf16x8 bh, bl;
        rows_bf16_split(st, hs, bh, bl);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const bf16x8 a = tr16_operand<D>(Kr, 32 * dt, 32 * t + 16 * hs, lane);
          acc[dt] = mma(a, bh, acc[dt]);
          acc[dt] = mma(a, bl, acc[dt]);
        }
      }
    }
  }
  store_cols<D>(dq + qoff, acc, scale, h);
}

// dk = scale * dS^T Q and dv = P^T dO, summed over the query heads of the kv head and
// the query blocks at or after the key block.  S = Q K^T here (a lane's column is a key).
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void k_attn_bwd_dkdv(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v, const float* __restrict__ lse,
                                                      const uint16_t* __restrict__ dO, const float* __restrict__ dsum,
                                                      int64_t T, int nh, int nkv, int64_t S, float scale, float sl2e,
                                                      uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                                                      float* __restrict__ part) {
  constexpr int QS = D + 8, NT = 64 * NW, BR = 32 * NW;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[BQ * QS];
  __shared__ __attribute__((aligned(16))) uint16_t Os[BQ * QS];   // dO rows
  __shared__ __attribute__((aligned(16))) uint16_t Qr[BQ * D];  // row-major, swizzled
  __shared__ __attribute__((aligned(16))) uint16_t Or[BQ * D];  // dO rows, row-major, swizzled
  __shared__ __attribute__((aligned(16))) float lse_s[BQ];
  __shared__ __attribute__((aligned(16))) float dsum_s[BQ];
  const int nqb = (int)(S / BQ), n_seq = (int)(T / S);
  const int seq = blockIdx.x % n_seq, kb = (int)(blockIdx.x / n_seq);  // early key blocks have the most work
  // part == nullptr: blockIdx.y is a kv head and the workgroup sums its query heads;
  // otherwise blockIdx.y is a query head and the workgroup writes that head's fp32 share
  const int rep = nh / nkv;
  const int hk = part ? (int)blockIdx.y / rep : (int)blockIdx.y;
  const int hq0 = part ? (int)blockIdx.y : hk * rep, hq1 = part ? hq0 + 1 : hk * rep + rep;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l32 = lane & 31, h = lane >> 5;
  const int64_t ldq = (int64_t)nh * D, ldk = (int64_t)nkv * D, t0 = (int64_t)seq * S;
  const int kpos = kb * BR + wave * 32 + l32;  // this lane's key
  const int qb_first = kb * BR / BQ;           // the first query block that sees these keys

  bf16x8 kf[D / 16], vf[D / 16];
  const int64_t koff = (t0 + kpos) * ldk + (int64_t)hk * D;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    kf[s] = ld16(k + koff + 16 * s + 8 * h);
    vf[s] = ld16(v + koff + 16 * s + 8 * h);
  }
  floatx16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    dka[dt] = zero16();
    dva[dt] = zero16();
  }

  Staged<D, NT> pq, po;
  pq.load(q, t0 + (int64_t)qb_first * BQ, ldq, (int64_t)hq0 * D);
  po.load(dO, t0 + (int64_t)qb_first * BQ, ldq, (int64_t)hq0 * D);
  // the block's per-query statistics travel with its rows: loaded one block ahead into
  // registers of the first BQ threads (a load issued just before the barrier that
  // publishes them would expose its latency once per block)
  float lse_n = 0.0f, dsum_n = 0.0f;
  if (threadIdx.x < BQ) {
    const int64_t r = (int64_t)hq0 * T + t0 + (int64_t)qb_first * BQ + threadIdx.x;
    lse_n = lse[r];
    dsum_n = dsum[r];
  }
  for (int hq = hq0; hq < hq1; ++hq)
    for (int qb = qb_first; qb < nqb; ++qb) {
      __syncthreads();
      pq.template rows<QS>(Qs);
      pq.rows_swz(Qr);
      po.template rows<QS>(Os);
      po.rows_swz(Or);
      if (threadIdx.x < BQ) {
        lse_s[threadIdx.x] = lse_n * 1.44269504088896341f;
        dsum_s[threadIdx.x] = dsum_n;
      }
      __syncthreads();
      {  // the next block (the next query block, or the next head's first) while this computes
        const bool last_qb = qb + 1 == nqb;
        if (!(last_qb && hq + 1 == hq1)) {
          const int nq = last_qb ? qb_first : qb + 1, nhq = last_qb ? hq + 1 : hq;
          pq.load(q, t0 + (int64_t)nq * BQ, ldq, (int64_t)nhq * D);
          po.load(dO, t0 + (int64_t)nq * BQ, ldq, (int64_t)nhq * D);
          if (threadIdx.x < BQ) {
            const int64_t r = (int64_t)nhq * T + t0 + (int64_t)nq * BQ + threadIdx.x;
            lse_n = lse[r];
            dsum_n = dsum[r];
          }
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        floatx16 sa = zero16(), dp = zero16();
        // the half block's Q and dO fragments are read into registers of their own before
        // the products (reused registers made every read wait for the MFMA before it)
        bf16x8 qa[D / 16], oa[D / 16];
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          qa[s] = ld16(&Qs[(32 * t + l32) * QS + 16 * s + 8 * h]);
          oa[s] = ld16(&Os[(32 * t + l32) * QS + 16 * s + 8 * h]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          sa = mma(qa[s], kf[s], sa);
          dp = mma(oa[s], vf[s], dp);
        }
        floatx16 ds;
        // a lane's 16 query rows come in 4 runs of 4 consecutive ones: one 16-byte read of
        // each statistic per run
        floatx4 lse4[4], dsum4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lse4[j] = *(const floatx4*)&lse_s[32 * t + 8 * j + 4 * h];
          dsum4[j] = *(const floatx4*)&dsum_s[32 * t + 8 * j + 4 * h];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qr = 32 * t + 8 * (i >> 2) + 4 * h + (i & 3);  // query row in the block
          // the exponential for every element, masked afterwards by a select: a branch
          // around it would split the wave's instruction stream 16 times per half block
          const float e = exp2f(sa[i] * sl2e - lse4[i >> 2][i & 3]);
          const float p = kpos > qb * BQ + qr ? 0.0f : e;
          sa[i] = p;
          ds[i] = p * (dp[i] - dsum4[i >> 2][i & 3]);
        }
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          bf16x8 ph, pl, sh, sl;
          rows_bf16_split(sa, hs, ph, pl);
          rows_bf16_split(ds, hs, sh, sl);
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            const bf16x8 ao = tr16_operand<D>(Or, 32 * dt, 32 * t + 16 * hs, lane);
            dva[dt] = mma(ao, ph, dva[dt]);
            dva[dt] = mma(ao, pl, dva[dt]);
            const bf16x8 a = tr16_operand<D>(Qr, 32 * dt, 32 * t + 16 * hs, lane);
            dka[dt] = mma(a, sh, dka[dt]);
            dka[dt] = mma(a, sl, dka[dt]);
          }
        }
      }
    }
  if (part == nullptr) {
    store_cols<D>(dk + koff, dka, scale, h);
    store_cols<D>(dv + koff, dva, 1.0f, h);
    return;
  }
  // fp32 shares: part[0][hq][t][d] for dk (scaled), part[1][hq][t][d] for dv
  const int64_t plane = (int64_t)nh * T * D;
  float* pk = part + ((int64_t)hq0 * T + t0 + kpos) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * dt + 8 * j + 4 * h;
      *(floatx4*)(pk + d0) = floatx4{dka[dt][4 * j] * scale, dka[dt][4 * j + 1] * scale, dka[dt][4 * j + 2] * scale,
                                     dka[dt][4 * j + 3] * scale};
      *(floatx4*)(pk + plane + d0) = floatx4{dva[dt][4 * j], dva[dt][4 * j + 1], dva[dt][4 * j + 2], dva[dt][4 * j + 3]};
    }
}

// dk, dv [T, n_kv * D] = bf16 of the sum over the rep query heads of each kv head, in
// head order
__global__ __launch_bounds__(256) void k_attn_bwd_kv_reduce(const float* __restrict__ part, int64_t T, int nh, int nkv,
                                                            int D, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
  const int rep = nh / nkv;
  const int64_t plane = (int64_t)nh * T * D, n4 = (int64_t)nkv * T * D / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const int64_t e = 4 * i;                       // element of [T, nkv, D]
    const int64_t t = e / ((int64_t)nkv * D);
    const int hk = (int)((e / D) % nkv);
    const int d = (int)(e % D);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < rep; ++j)
        acc += *(const floatx4*)(part + w * plane + ((int64_t)(hk * rep + j) * T + t) * D + d);
      uint2 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      *(uint2*)((w ? dv : dk) + e) = o;
    }
  }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t T, int nh, int nkv, int D,
                           int64_t S, uint16_t* o, float* lse, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const float sl2e = (float)(1.4426950408889634 / sqrt((double)D));
  const bool w4 = S % 128 == 0;
  const dim3 grid((unsigned)((S / (w4 ? 128 : 64)) * (T / S)), (unsigned)nh), block(w4 ? 256 : 128);
#define LNF4_FWD(D_, NW_) hipLaunchKernelGGL((k_attn_fwd<D_, NW_>), grid, block, 0, s, q, k, v, T, nh, nkv, S, sl2e, o, lse)
  if (D == 128) {
    if (w4) LNF4_FWD(128, 4); else LNF4_FWD(128, 2);
  } else {
    if (w4) LNF4_FWD(64, 4); else LNF4_FWD(64, 2);
  }
#undef LNF4_FWD
  return hipGetLastError();
}

size_t attn_bwd_workspace_bytes(int64_t T, int nh, int nkv, int D) {
  const size_t dsum = (size_t)nh * T * 4;
  const size_t part = nh == nkv ? 0 : 2 * (size_t)nh * T * D * 4;
  return ((dsum + 255) & ~(size_t)255) + part;
}

hipError_t launch_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                           const float* lse, const uint16_t* dO, int64_t T, int nh, int nkv, int D, int64_t S,
                           uint16_t* dq, uint16_t* dk, uint16_t* dv, void* workspace, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const float scale = (float)(1.0 / sqrt((double)D));
  const float sl2e = (float)(1.4426950408889634 / sqrt((double)D));  // as in the forward
  float* dsum = (float*)workspace;
  // with grouped kv heads every query head writes an fp32 share of dk, dv (4x the
  // workgroups of one per kv head), summed afterwards in head order
  float* part = nh == nkv ? nullptr : (float*)((uint8_t*)workspace + (((size_t)nh * T * 4 + 255) & ~(size_t)255));
  hipLaunchKernelGGL(k_attn_bwd_dsum, dim3((unsigned)(T < 65536 ? T : 65536)), dim3(256), 0, s, o, dO, T, nh, D, dsum);
  const bool w4 = S % 128 == 0;
  const int br = w4 ? 128 : 64;
  const dim3 gq((unsigned)((S / br) * (T / S)), (unsigned)nh);
  const dim3 gk((unsigned)((S / br) * (T / S)), (unsigned)(part ? nh : nkv));
  const dim3 block(w4 ? 256 : 128);
#define LNF4_BWD(D_, NW_)                                                                                   \
  hipLaunchKernelGGL((k_attn_bwd_dq<D_, NW_>), gq, block, 0, s, q, k, v, lse, dO, dsum, T, nh, nkv, S, scale, \
                     sl2e, dq);                                                                              \
  hipLaunchKernelGGL((k_attn_bwd_dkdv<D_, NW_>), gk, block, 0, s, q, k, v, lse, dO, dsum, T, nh, nkv, S,      \
                     scale, sl2e, dk, dv, part)
  if (D == 128) {
    if (w4) { LNF4_BWD(128, 4); } else { LNF4_BWD(128, 2); }
  } else {
    if (w4) { LNF4_BWD(64, 4); } else { LNF4_BWD(64, 2); }
  }
#undef LNF4_BWD
  if (part) {
    const int64_t n4 = (int64_t)nkv * T * D / 4;
    const int64_t b = (n4 + 255) / 256;
    hipLaunchKernelGGL(k_attn_bwd_kv_reduce, dim3((unsigned)(b < 8192 ? b : 8192)), dim3(256), 0, s, part, T, nh, nkv,
                       D, dk, dv);
  }
  return hipGetLastError();
}

}  // namespace lnf4
