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
// 32x32.  The activation tile (x or dy) is staged through LDS (a ring of 3 or 4 stages
// filled by direct-to-LDS loads, 16-byte chunks XOR-swizzled by row).  The K order inside a 64-wide step is permuted so that a
// lane's B fragments for the four 16-wide MFMA steps are 32 consecutive K values: lane
// (n, h) of a 32x32x16 MFMA supplies K = 32h + 8s .. 32h + 8s + 7 at step s.  Both
// operands use the same permutation, so the sum is unchanged.
//
//  * Forward: K runs along a row of W, so each lane loads its own 16 bytes of codes
//    (32 K values of one output column) straight from global memory into registers and
//    decodes them there: no LDS round trip for W, and every code is decoded once per
//    workgroup.  The decoded weights are the MFMA's A operand and the activations its B
//    operand, so the accumulators hold the tile transposed: a lane's consecutive
//    accumulator rows are adjacent outputs of one token, stored 8 bytes at a time.
//  * dx: K runs across rows of W (W is N-contiguous here).  The weight tile goes to LDS
//    row-major by direct loads and is read back transposed by gfx950's transposing LDS
//    reads (4-bit for the codes, which are then decoded in registers with each row's
//    absmax; 16-bit for bf16 weights), so each lane gets 8 consecutive K of one column.
//    For NF4 the decoded weights are again the A operand (transposed accumulators).
//  * Both NF4 kernels write their output through LDS: each wave stages its 64 columns of a
//    group of rows and stores whole 128-byte lines of the output.
#include "common.hpp"
#include "kernels.hpp"

namespace lnf4 {

__constant__ float c_gemm_table[16] = LNF4_TABLE_INIT;

constexpr int BN = 256;
constexpr int BK = 64;
constexpr int NTHR = 256;
constexpr int kGroupM = 4;   // row-tiles per group of the tile order (tile_coords)

// largest rank (summed over a group in backward) the fused epilogue stages in LDS
#define LNF4_EPI_RANK 64


// 16-byte-segment swizzle of a 128-byte code row (consecutive row pairs share it, so 16
// consecutive rows cover all 64 banks in a transposing read)
__device__ __forceinline__ int wswz(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ floatx16 mfma32(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint4 v = make_uint4(a, b, c, d);
  return __builtin_bit_cast(bf16x8, v);
}

// Activation tiles are [rows][64] bf16 (128-byte rows of eight 16-byte chunks).  Chunk c
// of row `row` sits at slot c ^ swz(row): with 64 LDS banks (256 bytes), the 16 lanes
// served together read rows r..r+15 at one logical chunk, and the even and the odd rows
// each cover 8 distinct slots, so a 16-byte-per-lane read is conflict free.
__device__ __forceinline__ int act_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int act_pos(int row, int c) { return row * BK + ((c ^ act_swz(row)) << 3); }

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
  LNF4_SEL(P, a.p, idx, part_off);
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
  LNF4_SEL(P, a.p, idx, v_stride);
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
// TR: the accumulators hold the transposed tile (MFMA A operand = adapter rows, B = U).
template <int MI, bool TR = false>
__device__ __forceinline__ void rank_update(floatx16 (&acc)[MI][2], const uint16_t* Uh, const uint16_t* Ul,
                                            const uint16_t* V, int RP, int l32, int h, int nc0, int nc1,
                                            int row0 = 0) {
  for (int ks = 0; ks < RP; ks += 16) {
    const bf16x8 b0 = *(const bf16x8*)&V[nc0 * RP + ks + 8 * h];
    const bf16x8 b1 = *(const bf16x8*)&V[nc1 * RP + ks + 8 * h];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = row0 + 32 * i + l32;
      const bf16x8 ah = *(const bf16x8*)&Uh[row * RP + ks + 8 * h];
      const bf16x8 al = *(const bf16x8*)&Ul[row * RP + ks + 8 * h];
      if (TR) {
        acc[i][0] = mfma32(b0, ah, acc[i][0]);
        acc[i][1] = mfma32(b1, ah, acc[i][1]);
        acc[i][0] = mfma32(b0, al, acc[i][0]);
        acc[i][1] = mfma32(b1, al, acc[i][1]);
      } else {
        acc[i][0] = mfma32(ah, b0, acc[i][0]);
        acc[i][1] = mfma32(ah, b1, acc[i][1]);
        acc[i][0] = mfma32(al, b0, acc[i][0]);
        acc[i][1] = mfma32(al, b1, acc[i][1]);
      }
    }
  }
}

__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  const __bf16 h = (__bf16)v;
  const __bf16 l = (__bf16)(v - (float)h);
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, l);
}


// =====================================================================================
// Forward
// =====================================================================================
// wait until at most n vector-memory ops of this wave are outstanding (gfx9 s_waitcnt
// encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at "no wait")
#define LNF4_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
// ... and every LDS access of this wave completed (lgkmcnt 0)
#define LNF4_WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4))

// The weight words one lane needs for one K-block: 32 codes (its K half) of each of its two
// columns, and the two columns' absmax of the block.
struct CodeSet {
  u32x4 w0, w1;
  float a0, a1;
};

// NF4 forward.  A lane's B fragments need only its own 16 code bytes per column and
// K-block, plus the block's absmax, so those come straight from global memory into
// registers three K-blocks ahead; only the activation tile goes through LDS, in a 4-stage
// ring.  Each 16-wide K step is split into two halves of MFMAs: the first half issues the
// next step's code-table and activation reads (and a third of the loads for the block
// three ahead), the second half the next fragments' fp32 products and bf16 packs.
// NW = 4: each wave owns 64 columns x all BM rows (one wave per SIMD).  The tile also
// compiles for NW = 8 (two waves per column group, each on half of the rows, two waves
// per SIMD, each code decoded by both); the launcher no longer uses it, since it measured
// slower than NW = 4 even for grids of under one tile per compute unit.
// LDS bytes of one ring stage: an activation tile, or (LoRA staging before the K loop,
// spread over three stages: hi, lo, adapter rows) a 64-rank slab
constexpr int fwd_stage_bytes(int BM) {
  return BM * BK * 2 > BN * LNF4_EPI_RANK * 2 ? BM * BK * 2 : BN * LNF4_EPI_RANK * 2;
}

// One BM x 256 output tile (tm, tn); sm0..sm3 are the ring stages (fwd_stage_bytes(BM)
// each), lut2 the byte-pair code table, filled by the caller.
template <int BM, int NW>
__device__ __forceinline__ void fwd_nf4_tile(const FwdArgs& args, int tm, int tn, uint8_t* sm0, uint8_t* sm1,
                                             uint8_t* sm2, uint8_t* sm3, const float2* lut2, int split = 0) {
  constexpr int NT = 64 * NW;
  constexpr int WM = NW / 4;          // waves sharing a column group
  constexpr int MI = BM / 32 / WM;    // 32-row MFMA tiles per wave
  constexpr int MH = MI / 2;          // MFMA rows of the first half-step
  constexpr int X_BYTES = BM * BK * 2;
  static_assert(MI % 2 == 0, "two half-steps");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int wn = wave & 3;                    // column group
  const int rbase = (wave >> 2) * (BM / WM);  // first tile row of this wave

  int pi = 0;
#pragma unroll
  for (int q = 1; q < kMaxGroup; ++q)
    if (q < args.n_proj && tn >= args.p[q].tile_n0) pi = q;
  const FwdProj P = select_fwd(args, pi);

  const int M = args.M, K = args.K, out_f = P.out_f;
  const int m0 = tm * BM;
  const int nloc0 = (tn - P.tile_n0) * BN;
  // K range of this split (the whole K when the launch is not split): the activation, code
  // and absmax resources start at its first K-block, so the loop below runs over nk blocks
  // as for an unsplit tile
  const bool splitk = args.ksplit > 1;
  const int kbs = splitk ? split * args.kb_per_split : 0;
  const int nk = splitk ? min(args.kb_per_split, K / BK - kbs) : K / BK;
  const int nc0 = 64 * wn + l32, nc1 = nc0 + 32;   // this lane's two tile columns

  // ---- accumulators start at the rank-r LoRA term s * u[m, :] . B[n, :]
  floatx16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  if (P.u != nullptr && P.r > 0 && kbs == 0) {  // the first split carries the LoRA term
    const int r = P.r, RP = (r + 15) & ~15;
    uint16_t* Uh = (uint16_t*)sm0;
    uint16_t* Ul = (uint16_t*)sm1;
    uint16_t* V = (uint16_t*)sm2;
    for (int idx = tid; idx < BM * RP; idx += NT) {
      const int mm = idx / RP, kk = idx - mm * RP, gm = m0 + mm;
      const float uv = (gm < M && kk < r) ? P.scale * P.u[(size_t)gm * r + kk] : 0.0f;
      split_bf16(uv, Uh[idx], Ul[idx]);
    }
    for (int idx = tid; idx < BN * RP; idx += NT) {
      const int nn = idx / RP, kk = idx - nn * RP, n = nloc0 + nn;
      V[idx] = (n < out_f && kk < r) ? P.B[(size_t)n * r + kk] : (uint16_t)0;
    }
    __syncthreads();
    rank_update<MI, true>(acc, Uh, Ul, V, RP, l32, h, nc0, nc1, rbase);
    __syncthreads();
  }

  // ---- activation stream (LDS).  Every direct load of a wave writes 64 consecutive
  // 16-byte LDS slots, lane L to slot L: load q of wave w fills tile rows (w*XQ+q)*8 .. +7,
  // lane L holds row (w*XQ+q)*8 + L/8, slot L%8 = logical chunk (L%8) ^ swz(row).  Rows >= M
  // read row M-1 (their outputs are discarded).  A 32-bit per-lane offset plus the K-block
  // advance as the wave-uniform offset: no per-lane address arithmetic in the K loop.
  constexpr int XQ = X_BYTES / 1024 / NW;
  static_assert(XQ % 2 == 0, "activation loads split over two steps");
  constexpr int NLD = XQ + 4;  // vector-memory ops per wave per K-block
  const rsrc_t xrs = make_rsrc(args.x + (size_t)m0 * K + (size_t)kbs * BK, (int64_t)(M - m0) * K * 2 - (int64_t)kbs * BK * 2);
  uint32_t xoff[XQ];
#pragma unroll
  for (int q = 0; q < XQ; ++q) {
    const int row = (wave * XQ + q) * 8 + (lane >> 3);
    const int lr = (m0 + row < M) ? row : (M - 1 - m0);
    xoff[q] = 2u * ((uint32_t)lr * (uint32_t)K + (uint32_t)(((lane & 7) ^ act_swz(row)) * 8));
  }
  // ---- weight words (registers): codes of columns nc0 / nc1, K half h; columns >= out_f
  // read column out_f - 1 (their outputs are discarded)
  const rsrc_t wrs = make_rsrc((const uint8_t*)P.w + (size_t)kbs * 32, (int64_t)out_f * K / 2 - (int64_t)kbs * 32);
  const rsrc_t ars = make_rsrc(P.absmax + kbs, ((int64_t)out_f * (K / 64) - kbs) * 4);
  const int g0 = nloc0 + nc0 < out_f ? nloc0 + nc0 : out_f - 1;
  const int g1 = nloc0 + nc1 < out_f ? nloc0 + nc1 : out_f - 1;
  const uint32_t woff0 = (uint32_t)g0 * (uint32_t)(K / 2) + 16u * h;
  const uint32_t woff1 = (uint32_t)g1 * (uint32_t)(K / 2) + 16u * h;
  const uint32_t aoff0 = 4u * (uint32_t)g0 * (uint32_t)(K / 64);
  const uint32_t aoff1 = 4u * (uint32_t)g1 * (uint32_t)(K / 64);

#define LNF4_Q_XLOAD(kb_, SM_, part_)                                                        \
  _Pragma("unroll") for (int q = (part_) * (XQ / 2); q < ((part_) + 1) * (XQ / 2); ++q)      \
      LNF4_BUF_LDS(xrs, (SM_) + (wave_u * XQ + q) * 1024, 16, xoff[q], (kb_) * (BK * 2));
  // Blocks past the last (the loop runs whole trips of 8 blocks) read absmax 0 through an
  // out-of-range offset (the buffer load returns zero), so their decoded weights are zeros.
#define LNF4_Q_WLOAD(kb_, CS_)                                                               \
  {                                                                                          \
    const int kw_ = (kb_) < nk ? (kb_) : nk - 1;                                             \
    CS_.w0 = LNF4_BUF_LD128(wrs, woff0, kw_ * 32);                                           \
    CS_.w1 = LNF4_BUF_LD128(wrs, woff1, kw_ * 32);                                           \
    CS_.a0 = __uint_as_float(LNF4_BUF_LD32(ars, (kb_) < nk ? aoff0 : 0x7fff0000u, kw_ * 4));  \
    CS_.a1 = __uint_as_float(LNF4_BUF_LD32(ars, (kb_) < nk ? aoff1 : 0x7fff0000u, kw_ * 4));  \
  }
  // NF4 B fragment (8 consecutive K of one column): table-read phase (byte -> LDS table ->
  // fp32 levels of its two codes) and finish phase (one fp32 product by the block's absmax,
  // RNE pack to bf16), exactly the standalone decode
#define LNF4_LUT8(lv, cw_)                                                         \
  {                                                                                \
    const uint32_t c_ = (cw_);                                                     \
    _Pragma("unroll") for (int b_ = 0; b_ < 4; ++b_) {                             \
      const float2 p_ = lut2[(c_ >> (8 * b_)) & 255u];                             \
      lv[2 * b_] = p_.x;                                                           \
      lv[2 * b_ + 1] = p_.y;                                                       \
    }                                                                              \
  }
#define LNF4_FIN8(dst, lv, a_)                                                     \
  dst = as_bf16x8(pack_bf16x2(lv[0] * (a_), lv[1] * (a_)), pack_bf16x2(lv[2] * (a_), lv[3] * (a_)), \
                  pack_bf16x2(lv[4] * (a_), lv[5] * (a_)), pack_bf16x2(lv[6] * (a_), lv[7] * (a_)));
#define LNF4_XS(SM_) ((const uint16_t*)(SM_))
#define LNF4_AFRAG(SM_, i_, chunk_) (*(const bf16x8*)&LNF4_XS(SM_)[act_pos(rbase + 32 * (i_) + l32, (chunk_))])

  // prologue: blocks 0, 1, 2 in flight (activations, then weight words, block by block);
  // block 0 visible
  CodeSet k0, k1, k2, k3;
  LNF4_Q_XLOAD(0, sm0, 0);
  LNF4_Q_XLOAD(0, sm0, 1);
  LNF4_Q_WLOAD(0, k0);
  LNF4_Q_XLOAD((nk > 1 ? 1 : nk - 1), sm1, 0);
  LNF4_Q_XLOAD((nk > 1 ? 1 : nk - 1), sm1, 1);
  LNF4_Q_WLOAD(1, k1);
  LNF4_Q_XLOAD((nk > 2 ? 2 : nk - 1), sm2, 0);
  LNF4_Q_XLOAD((nk > 2 ? 2 : nk - 1), sm2, 1);
  LNF4_Q_WLOAD(2, k2);
  LNF4_WAIT_VM(2 * NLD);
  __syncthreads();

  bf16x8 ac[MI], an_[MI];
  bf16x8 bc0, bc1, bn0, bn1;
  {
    float l0[8], l1[8];
    LNF4_LUT8(l0, k0.w0[0]);
    LNF4_LUT8(l1, k0.w1[0]);
    LNF4_FIN8(bc0, l0, k0.a0);
    LNF4_FIN8(bc1, l1, k0.a1);
  }
#pragma unroll
  for (int i = 0; i < MI; ++i) ac[i] = LNF4_AFRAG(sm0, i, 4 * h);

  // One K-block KB: stage SC holds it, SN the next one, SP receives the block three ahead;
  // CC / CN are the weight words of this block / the next, CL receives those of the block
  // three ahead.
#define LNF4_Q_BLOCK(KB, SC, SN, SP, CC, CN, CL)                                               \
  {                                                                                            \
    const int kl_ = (KB) + 3 < nk ? (KB) + 3 : nk - 1; /* past the end: re-read the last */    \
    _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                            \
      __builtin_amdgcn_sched_barrier(0);                                                       \
      if (s == 3) {                                                                            \
        /* block KB+1 in LDS for every wave, and every wave done with stage SC before */      \
        /* block KB+4 is issued into it (a bare s_barrier: a fenced __syncthreads would */     \
        /* also wait for the loads of blocks KB+2 and KB+3, which are meant to stay in */     \
        /* flight) */                                                                          \
        LNF4_WAIT_VM_LGKM0(2 * NLD);                                                           \
        __builtin_amdgcn_s_barrier();                                                          \
        __builtin_amdgcn_sched_barrier(0);                                                     \
      }                                                                                        \
      float l0[8], l1[8];                                                                      \
      LNF4_LUT8(l0, (s < 3 ? CC.w0[s + 1 < 4 ? s + 1 : 0] : CN.w0[0]));                        \
      LNF4_LUT8(l1, (s < 3 ? CC.w1[s + 1 < 4 ? s + 1 : 0] : CN.w1[0]));                        \
      _Pragma("unroll") for (int i = 0; i < MI; ++i) an_[i] =                                  \
          (s < 3) ? LNF4_AFRAG(SC, i, 4 * h + s + 1) : LNF4_AFRAG(SN, i, 4 * h);               \
      if (s < 2) { LNF4_Q_XLOAD(kl_, SP, s); }                                                 \
      if (s == 2) LNF4_Q_WLOAD((KB) + 3, CL);                                                  \
      _Pragma("unroll") for (int i = 0; i < MH; ++i) {                                         \
        acc[i][0] = mfma32(bc0, ac[i], acc[i][0]);                                             \
        acc[i][1] = mfma32(bc1, ac[i], acc[i][1]);                                             \
      }                                                                                        \
      /* first half: table addresses and reads, then activation reads and loads */            \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                       \
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);                                       \
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);                                       \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                       \
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);                                       \
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);                                       \
      _Pragma("unroll") for (int g = 2; g < 2 * MH; ++g) {                                     \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                     \
        __builtin_amdgcn_sched_group_barrier(0x100, MH > 1 ? (MI + 2 * MH - 3) / (2 * MH - 2) : 1, 0); \
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                                     \
      }                                                                                        \
      __builtin_amdgcn_sched_barrier(0);                                                       \
      _Pragma("unroll") for (int i = MH; i < MI; ++i) {                                        \
        acc[i][0] = mfma32(bc0, ac[i], acc[i][0]);                                             \
        acc[i][1] = mfma32(bc1, ac[i], acc[i][1]);                                             \
      }                                                                                        \
      LNF4_FIN8(bn0, l0, (s < 3 ? CC.a0 : CN.a0));                                             \
      LNF4_FIN8(bn1, l1, (s < 3 ? CC.a1 : CN.a1));                                             \
      /* second half: products and packs of the next fragments between the MFMAs */           \
      _Pragma("unroll") for (int g = 0; g < 2 * (MI - MH); ++g) {                              \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                     \
        __builtin_amdgcn_sched_group_barrier(0x002, (24 + 2 * (MI - MH) - 1) / (2 * (MI - MH)), 0); \
      }                                                                                        \
      /* with one wave per SIMD, the fragments this step's MFMAs read stay live to its end, */ \
      /* so the next step's fragments go to other registers: overwriting a register that an */ \
      /* MFMA in flight still reads stalls the wave (two waves per SIMD have no registers */   \
      /* to spare for it) */                                                                   \
      if (NW == 4) {                                                                           \
        asm volatile("" ::"v"(bc0), "v"(bc1));                                                 \
        _Pragma("unroll") for (int i = 0; i < MI; ++i) asm volatile("" ::"v"(ac[i]));          \
      }                                                                                        \
      _Pragma("unroll") for (int i = 0; i < MI; ++i) ac[i] = an_[i];                           \
      bc0 = bn0;                                                                               \
      bc1 = bn1;                                                                               \
    }                                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                         \
    /* the next block's first B fragments exist before the block ends: otherwise their */     \
    /* decode sinks into the next block and stalls its first MFMAs */                         \
    asm volatile("" ::"v"(bc0), "v"(bc1));                                                     \
  }

  // Whole trips over two turns of the 4-stage ring with one exit test per trip.  (With an
  // exit after every block, the compiler's wait-count merging at the loop exits inserted a
  // near-full drain of the loads in flight once per trip.)
  const int nk8 = (nk + 7) & ~7;
  for (int kb = 0; kb < nk8; kb += 8) {
    LNF4_Q_BLOCK(kb + 0, sm0, sm1, sm3, k0, k1, k3);
    LNF4_Q_BLOCK(kb + 1, sm1, sm2, sm0, k1, k2, k0);
    LNF4_Q_BLOCK(kb + 2, sm2, sm3, sm1, k2, k3, k1);
    LNF4_Q_BLOCK(kb + 3, sm3, sm0, sm2, k3, k0, k2);
    LNF4_Q_BLOCK(kb + 4, sm0, sm1, sm3, k0, k1, k3);
    LNF4_Q_BLOCK(kb + 5, sm1, sm2, sm0, k1, k2, k0);
    LNF4_Q_BLOCK(kb + 6, sm2, sm3, sm1, k2, k3, k1);
    LNF4_Q_BLOCK(kb + 7, sm3, sm0, sm2, k3, k0, k2);
  }
#undef LNF4_Q_BLOCK
#undef LNF4_Q_XLOAD
#undef LNF4_Q_WLOAD
#undef LNF4_LUT8
#undef LNF4_FIN8
#undef LNF4_XS
#undef LNF4_AFRAG

  // ---- K split: this split's fp32 sums, added up by a second launch in split order.  As for
  // the bf16 output below, each wave stages its 64 columns of its rows in its column group's
  // ring stage (a row is 256 bytes: 16-byte chunk c at c ^ (row & 15), so the 32 rows one
  // staging write covers spread over all banks) and then stores whole 256-byte row pieces,
  // 16 lanes to a row; rows that do not fit the stage at once (256-row tiles) go in passes.
  if (splitk) {
    LNF4_WAIT_VM_LGKM0(0);  // the ring's last (past-the-end) loads have landed
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    uint8_t* const stg = wn == 0 ? sm0 : (wn == 1 ? sm1 : (wn == 2 ? sm2 : sm3));
    constexpr int RPW = BM / WM;                                   // rows of this wave
    constexpr int RPP = RPW < fwd_stage_bytes(BM) / 256 ? RPW : fwd_stage_bytes(BM) / 256;  // per pass
    static_assert(RPW % RPP == 0 && RPP % 32 == 0, "whole MFMA row blocks per pass");
    float* const pp = args.part + P.part_off + (size_t)split * M * out_f;
    const int cl = lane & 15;
    const int n = nloc0 + 64 * wn + 4 * cl;
#pragma unroll
    for (int pass = 0; pass < RPW / RPP; ++pass) {
#pragma unroll
      for (int i = pass * (RPP / 32); i < (pass + 1) * (RPP / 32); ++i) {
        const int row = 32 * i + l32 - pass * RPP;  // row within the pass
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = 8 * j + 2 * g + h;
            *(floatx4*)(stg + row * 256 + ((c ^ (row & 15)) * 16)) =
                floatx4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging writes are done
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < RPP / 4; ++k) {
        const int row = 4 * k + (lane >> 4);
        const floatx4 v = *(const floatx4*)(stg + row * 256 + ((cl ^ (row & 15)) * 16));
        const int gm = m0 + rbase + pass * RPP + row;
        if (gm < M && n < out_f) *(floatx4*)(pp + (size_t)gm * out_f + n) = v;
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // the pass's reads are done before the next overwrites
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }
  // ---- store bf16.  The accumulators hold the transposed tile: lane (l32, h) has token
  // rbase + 32i + l32 and, for q = 4g..4g+3, the four adjacent outputs 32j + 8g + 4h + 0..3
  // of its column group.  Each wave's 64 columns of a row are one 128-byte line of y, so the
  // wave stages its rows in LDS (its column group's ring stage, free once every wave is past
  // its last K-block: 16-byte chunk c of row r at c ^ ((r >> 1) & 7)) and writes whole lines,
  // 16 bytes per lane, 8 rows per store: scattered 8-byte stores to 32 rows each cost the
  // memory pipeline far more (about 10 us of a 115 us tile at the 8B gate|up shape).
  if ((out_f & 7) == 0 && (((uintptr_t)P.y) & 15) == 0) {
    LNF4_WAIT_VM_LGKM0(0);  // the ring's last (past-the-end) loads have landed
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    uint8_t* const stg = wn == 0 ? sm0 : (wn == 1 ? sm1 : (wn == 2 ? sm2 : sm3));
    uint8_t* const rg = stg + rbase * 128;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = 32 * i + l32;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int pc = (4 * j + g) ^ ((row >> 1) & 7);
          *(uint2*)(rg + row * 128 + pc * 16 + 8 * h) =
              make_uint2(pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                         pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]));
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging writes are done
    __builtin_amdgcn_sched_barrier(0);
    const int c = lane & 7;
    const int n = nloc0 + 64 * wn + 8 * c;
#pragma unroll
    for (int k = 0; k < BM / WM / 8; ++k) {
      const int row = 8 * k + (lane >> 3);
      const u32x4 v = *(const u32x4*)(rg + row * 128 + ((c ^ ((row >> 1) & 7)) * 16));
      const int gm = m0 + rbase + row;
      if (gm < M && n < out_f) *(u32x4*)(P.y + (size_t)gm * out_f + n) = v;
    }
    return;
  }
  const bool vec4 = (out_f & 3) == 0 && (((uintptr_t)P.y) & 7) == 0;  // y need only be 2-byte aligned
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    __builtin_amdgcn_sched_barrier(0);  // bound the accumulator reads that are live at once
    const int gm = m0 + rbase + 32 * i + l32;
    if (gm >= M) continue;
    uint16_t* yr = P.y + (size_t)gm * out_f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = nloc0 + 64 * wn + 32 * j + 8 * g + 4 * h;
        const float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        if (vec4 && n < out_f) {
          *(uint2*)(yr + n) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < out_f) yr[n + e] = __builtin_bit_cast(uint16_t, (__bf16)v[e]);
        }
      }
  }
}

// Blocks compute BM-row tiles over n_tiles_m x n_tiles_n.  With BM = 256 and 4 waves, a
// tail of 128-row tiles over the tail_n column panels that follow can be mixed in: a last
// round of tiles that would leave compute units idle runs as twice as many half-height
// tiles.  When the tail is one round, four of the eight XCDs run their tail tiles first, so
// those XCDs are half a tile out of step with the other four and the output stores at the
// end of each tile do not all hit memory at once.
template <int BM, int NW>
__global__ __launch_bounds__(64 * NW, 1) void k_fwd_nf4(const FwdArgs args) {
  constexpr int STAGE = fwd_stage_bytes(BM);
  static_assert(4 * STAGE + 2048 <= 160 * 1024, "LDS budget");
  static_assert(fwd_stage_bytes(128) <= STAGE, "128-row tiles share the ring");
  // four distinct LDS objects, one per ring stage: the compiler then knows which
  // direct-to-LDS loads each LDS read can alias and never waits for the loads still
  // streaming into the other stages
  __shared__ __attribute__((aligned(16))) uint8_t sm0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm2[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm3[STAGE];
  // byte-pair code table: entry b = (T[b >> 4], T[b & 15]), the fp32 levels of the two
  // codes one byte holds (high nibble first)
  __shared__ __attribute__((aligned(2048))) float2 lut2[256];
  const int tid = threadIdx.x;
  if (tid < 256) lut2[tid] = make_float2(c_gemm_table[tid >> 4], c_gemm_table[tid & 15]);

  int tm, tn;
  const int b = blockIdx.x;
  if (args.ksplit > 1) {
    // K splits: blocks [s T, (s+1) T) run split s of the T = n_tiles_m x n_tiles_n tiles
    const int nt = args.n_tiles_m * args.n_tiles_n, sp = b / nt;
    tile_coords(b - sp * nt, args.n_tiles_m, args.n_tiles_n, kGroupM, tm, tn);
    fwd_nf4_tile<BM, NW>(args, tm, tn + args.tn_base, sm0, sm1, sm2, sm3, lut2, sp);
    return;
  }
  if constexpr (BM == 256 && NW == 4) {
    if (args.xcd_f > 0) {
      // XCD x = b mod 8 runs its blocks i = b / 8 in order; its tiles are the contiguous
      // ranges [x xcd_f, (x+1) xcd_f) of the full-tile sequence and [x xcd_h, (x+1) xcd_h)
      // of the tail sequence, as tile_coords would give it
      const int x = b & 7, i = b >> 3;
      const bool tail_first = x >= 4;
      const int n_first = tail_first ? args.xcd_h : args.xcd_f;
      const bool is_tail = tail_first ? i < n_first : i >= n_first;
      const int j = i < n_first ? i : i - n_first;
      if (is_tail) {
        tile_from_seq(args.xcd_h * x + j, args.tail_m, args.tail_n, kGroupM, tm, tn);
        fwd_nf4_tile<128, 4>(args, tm, tn + args.tn_base + args.n_tiles_n, sm0, sm1, sm2, sm3, lut2);
      } else {
        tile_from_seq(args.xcd_f * x + j, args.n_tiles_m, args.n_tiles_n, kGroupM, tm, tn);
        fwd_nf4_tile<BM, NW>(args, tm, tn + args.tn_base, sm0, sm1, sm2, sm3, lut2);
      }
      return;
    }
    if (b >= args.split_block) {
      tile_coords(b - args.split_block, args.tail_m, args.tail_n, kGroupM, tm, tn);
      fwd_nf4_tile<128, 4>(args, tm, tn + args.tn_base + args.n_tiles_n, sm0, sm1, sm2, sm3, lut2);
      return;
    }
  }
  tile_coords(b, args.n_tiles_m, args.n_tiles_n, kGroupM, tm, tn);
  fwd_nf4_tile<BM, NW>(args, tm, tn + args.tn_base, sm0, sm1, sm2, sm3, lut2);
}

// bf16 weights: the weight tile goes through LDS beside the activation tile (128 bytes per
// column and K-block, 16-byte chunks swizzled like the activation rows), in a 3-stage ring;
// its 4x larger weight tiles only fit LDS with 128-row tiles.  Wave w owns the 64 columns
// [64w, 64w+64) and all BM rows.
template <int BM>
__global__ __launch_bounds__(NTHR, 1) void k_fwd_bf16(const FwdArgs args) {
  constexpr int MI = BM / 32;
  constexpr int NM = 2 * MI;                       // MFMAs per 16-wide K step
  constexpr int X_BYTES = BM * BK * 2;
  constexpr int W_BYTES = BN * 128;
  constexpr int STAGE_RAW = X_BYTES + W_BYTES;
  constexpr int EPI_SLAB = BN * LNF4_EPI_RANK * 2;
  constexpr int STAGE = STAGE_RAW > EPI_SLAB ? STAGE_RAW : EPI_SLAB;
  static_assert(3 * STAGE <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint8_t sm0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm2[STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  int tm, tn;
  tile_coords(blockIdx.x, args.n_tiles_m, args.n_tiles_n, kGroupM, tm, tn);
  tn += args.tn_base;
  int pi = 0;
#pragma unroll
  for (int q = 1; q < kMaxGroup; ++q)
    if (q < args.n_proj && tn >= args.p[q].tile_n0) pi = q;
  const FwdProj P = select_fwd(args, pi);

  const int M = args.M, K = args.K, out_f = P.out_f;
  const int m0 = tm * BM;
  const int nloc0 = (tn - P.tile_n0) * BN;
  const int nk = K / BK;
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
    uint16_t* Uh = (uint16_t*)sm0;
    uint16_t* Ul = (uint16_t*)sm1;
    uint16_t* V = (uint16_t*)sm2;
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
    rank_update<MI, true>(acc, Uh, Ul, V, RP, l32, h, nc0, nc1);
    __syncthreads();
  }

  // global -> LDS streams, two K-blocks ahead (lane L of a direct load writes slot L):
  //  * activation: load q of wave w fills tile rows (w*XQ+q)*8 .. +7, as in the NF4 kernel;
  //  * weights: per column 128 bytes (8 chunks, swizzled like the activation rows); wave w
  //    loads columns 8g .. 8g+7 for g = w*WQ .. w*WQ+WQ-1, lane L -> column 8g + L/8.
  //  Columns >= out_f read column out_f-1 (outputs discarded).
  constexpr int XQ = X_BYTES / 1024 / 4;
  constexpr int WQ = 32 / 4;
  constexpr int NLD = XQ + WQ;
  const rsrc_t xrs = make_rsrc(args.x + (size_t)m0 * K, (int64_t)(M - m0) * K * 2);
  uint32_t xoff[XQ];
#pragma unroll
  for (int q = 0; q < XQ; ++q) {
    const int row = (wave * XQ + q) * 8 + (lane >> 3);
    const int lr = (m0 + row < M) ? row : (M - 1 - m0);
    xoff[q] = 2u * ((uint32_t)lr * (uint32_t)K + (uint32_t)(((lane & 7) ^ act_swz(row)) * 8));
  }
  const rsrc_t wrs = make_rsrc(P.w, (int64_t)out_f * K * 2);
  uint32_t woff[WQ];
#pragma unroll
  for (int q = 0; q < WQ; ++q) {
    const int col = 8 * (wave * WQ + q) + (lane >> 3);
    int n = nloc0 + col;
    n = n < out_f ? n : out_f - 1;
    woff[q] = (uint32_t)n * (uint32_t)K * 2u + (uint32_t)(((lane & 7) ^ act_swz(col)) * 16);
  }

#define LNF4_ISSUE(kb_, SM_)                                                                    \
  {                                                                                             \
    uint8_t* sx_ = SM_;                                                                         \
    _Pragma("unroll") for (int q = 0; q < XQ; ++q)                                              \
        LNF4_BUF_LDS(xrs, sx_ + (wave_u * XQ + q) * 1024, 16, xoff[q], (kb_) * (BK * 2));       \
    _Pragma("unroll") for (int q = 0; q < WQ; ++q)                                              \
        LNF4_BUF_LDS(wrs, sx_ + X_BYTES + (wave_u * WQ + q) * 1024, 16, woff[q], (kb_) * 128);  \
  }
  // chunk 4h+s of a column
#define LNF4_READ_BW(SM_, s_, col_) \
  (*(const bf16x8*)((SM_) + X_BYTES + (col_) * 128 + (((4 * h + (s_)) ^ act_swz(col_)) * 16)))
#define LNF4_XS(SM_) ((const uint16_t*)(SM_))

  // prologue: blocks 0 and 1 in flight; block 0 visible
  LNF4_ISSUE(0, sm0);
  LNF4_ISSUE((nk > 1 ? 1 : 0), sm1);
  LNF4_WAIT_VM(NLD);
  __syncthreads();

  bf16x8 ac[MI], an_[MI];
  bf16x8 bc0, bc1, bn0, bn1;
  bc0 = LNF4_READ_BW(sm0, 0, nc0);
  bc1 = LNF4_READ_BW(sm0, 0, nc1);
#pragma unroll
  for (int i = 0; i < MI; ++i) ac[i] = *(const bf16x8*)&LNF4_XS(sm0)[act_pos(32 * i + l32, 4 * h)];

  // One K-block on stage SC; SN holds the next block, SP receives the block two ahead.
  // The loop is unrolled three times with the stages rotated, so every LDS access names
  // its stage statically.
#define LNF4_FWD_BLOCK(SC, SN, SP)                                                             \
  {                                                                                            \
    _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                            \
      __builtin_amdgcn_sched_barrier(0);                                                       \
      if (s == 1) {                                                                            \
        /* block kb+2 goes into stage SP, which no wave reads any more.  Issued after step */  \
        /* 0's LDS reads: at the loop head the compiler cannot tell which stage an */         \
        /* in-flight load targets and drains them all before the first LDS read, and */       \
        /* that first read now only waits for block kb+1, issued a block ago */               \
        LNF4_ISSUE((kb + 2 < nk ? kb + 2 : nk - 1), SP); /* the tail re-reads the last block */ \
        __builtin_amdgcn_sched_barrier(0);                                                     \
      }                                                                                        \
      if (s == 3) {                                                                            \
        /* block kb+1 (issued one block ago) in LDS for every wave, and every wave done */     \
        /* with stage SC before block kb+3 is issued into it */                                \
        LNF4_WAIT_VM_LGKM0(NLD);                                                               \
        __builtin_amdgcn_s_barrier();                                                          \
        __builtin_amdgcn_sched_barrier(0);                                                     \
      }                                                                                        \
      if (s < 3) {                                                                             \
        bn0 = LNF4_READ_BW(SC, s + 1, nc0);                                                    \
        bn1 = LNF4_READ_BW(SC, s + 1, nc1);                                                    \
        _Pragma("unroll") for (int i = 0; i < MI; ++i) an_[i] =                                \
            *(const bf16x8*)&LNF4_XS(SC)[act_pos(32 * i + l32, 4 * h + s + 1)];                \
      } else {                                                                                 \
        bn0 = LNF4_READ_BW(SN, 0, nc0);                                                        \
        bn1 = LNF4_READ_BW(SN, 0, nc1);                                                        \
        _Pragma("unroll") for (int i = 0; i < MI; ++i) an_[i] =                                \
            *(const bf16x8*)&LNF4_XS(SN)[act_pos(32 * i + l32, 4 * h)];                        \
      }                                                                                        \
      _Pragma("unroll") for (int i = 0; i < MI; ++i) {                                         \
        acc[i][0] = mfma32(bc0, ac[i], acc[i][0]);                                             \
        acc[i][1] = mfma32(bc1, ac[i], acc[i][1]);                                             \
      }                                                                                        \
      _Pragma("unroll") for (int g = 0; g < NM; ++g) {                                         \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                     \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                     \
      }                                                                                        \
      _Pragma("unroll") for (int i = 0; i < MI; ++i) ac[i] = an_[i];                           \
      bc0 = bn0;                                                                               \
      bc1 = bn1;                                                                               \
    }                                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                         \
  }

  // unrolled twice over (six blocks per trip): the compiler drops the per-stage
  // knowledge of in-flight loads at the loop head and drains them there once per trip
  for (int kb = 0;;) {
    LNF4_FWD_BLOCK(sm0, sm1, sm2);
    if (++kb == nk) break;
    LNF4_FWD_BLOCK(sm1, sm2, sm0);
    if (++kb == nk) break;
    LNF4_FWD_BLOCK(sm2, sm0, sm1);
    if (++kb == nk) break;
    LNF4_FWD_BLOCK(sm0, sm1, sm2);
    if (++kb == nk) break;
    LNF4_FWD_BLOCK(sm1, sm2, sm0);
    if (++kb == nk) break;
    LNF4_FWD_BLOCK(sm2, sm0, sm1);
    if (++kb == nk) break;
  }
#undef LNF4_FWD_BLOCK
#undef LNF4_READ_BW
#undef LNF4_XS
#undef LNF4_ISSUE

  // ---- store bf16.  As in the NF4 forward the weights are the MFMA's A operand, so the
  // accumulators hold the tile transposed: lane (l32, h) has token 32i + l32 and, for
  // q = 4g..4g+3, the outputs 64 wave + 32j + 8g + 4h + 0..3.  With out_f % 8 == 0 and y
  // 16-byte aligned each wave stages its rows in LDS (16-byte chunk c of row r at
  // c ^ ((r >> 1) & 7), in the first two ring stages, free once every wave is past its last
  // K-block) and stores whole 128-byte lines; else 8-byte groups or single elements.
  if ((out_f & 7) == 0 && (((uintptr_t)P.y) & 15) == 0) {
    LNF4_WAIT_VM_LGKM0(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    uint8_t* const rg = (wave < 2 ? sm0 : sm1) + (wave & 1) * (BM * 128);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = 32 * i + l32;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int pc = (4 * j + g) ^ ((row >> 1) & 7);
          *(uint2*)(rg + row * 128 + pc * 16 + 8 * h) =
              make_uint2(pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                         pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]));
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging writes are done
    __builtin_amdgcn_sched_barrier(0);
    const int c = lane & 7;
    const int n = nloc0 + 64 * wave + 8 * c;
#pragma unroll
    for (int k = 0; k < BM / 8; ++k) {
      const int row = 8 * k + (lane >> 3);
      const u32x4 v = *(const u32x4*)(rg + row * 128 + ((c ^ ((row >> 1) & 7)) * 16));
      const int gm = m0 + row;
      if (gm < M && n < out_f) *(u32x4*)(P.y + (size_t)gm * out_f + n) = v;
    }
    return;
  }
  const bool vec4 = (out_f & 3) == 0 && (((uintptr_t)P.y) & 7) == 0;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    const int gm = m0 + 32 * i + l32;
    if (gm >= M) continue;
    uint16_t* yr = P.y + (size_t)gm * out_f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = nloc0 + 64 * wave + 32 * j + 8 * g + 4 * h;
        const float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        if (vec4 && n < out_f) {
          *(uint2*)(yr + n) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < out_f) yr[n + e] = __builtin_bit_cast(uint16_t, (__bf16)v[e]);
        }
      }
  }
}

// Forward, bf16 weights, 256-row tiles: 32-wide K-blocks in a 5-stage ring, as the
// 256-row input gradient.  Both operands are K-contiguous, so the activation tile [256][32]
// and the weight tile [256 columns][32] share one layout: 64-byte rows, 16-byte chunk c of
// row r at slot c ^ ((r >> 2) & 3) (the 16 rows one read phase serves cover all 16 bank
// groups).  Lane (n, h) of the MFMA supplies K = 16h + 8s .. +7 at step s.  The weights are
// the MFMA's A operand, so the accumulators hold the tile transposed, as in the 128-row
// kernel.  A block's activation rows are issued right after the barrier that frees its
// stage, its weight rows one step later.  Blocks past the last read the last block's
// activations against an empty weight range (zeros), so the loop runs whole turns of the
// ring.
__global__ __launch_bounds__(NTHR, 1) void k_fwd_bf16_deep(const FwdArgs args) {
  constexpr int BM = 256, MI = 8, NM = 16;
  constexpr int KS = 32;                    // K-block width
  constexpr int X_BYTES = BM * KS * 2;      // activation tile [256][32] bf16
  constexpr int W_BYTES = BN * KS * 2;      // weight tile [256][32] bf16
  constexpr int STAGE = X_BYTES + W_BYTES;  // 32 KB
  static_assert(BM * LNF4_EPI_RANK * 2 <= STAGE && BN * LNF4_EPI_RANK * 2 <= STAGE, "LoRA slabs fit a stage");
  static_assert(BM * 128 <= STAGE, "a wave's output rows fit a stage");
  static_assert(5 * STAGE <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint8_t sm0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm2[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm3[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm4[STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  int tm, tn;
  tile_coords(blockIdx.x, args.n_tiles_m, args.n_tiles_n, kGroupM, tm, tn);
  tn += args.tn_base;
  int pi = 0;
#pragma unroll
  for (int q = 1; q < kMaxGroup; ++q)
    if (q < args.n_proj && tn >= args.p[q].tile_n0) pi = q;
  const FwdProj P = select_fwd(args, pi);

  const int M = args.M, K = args.K, out_f = P.out_f;
  const int m0 = tm * BM;
  const int nloc0 = (tn - P.tile_n0) * BN;
  const int nk = K / KS;
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
    uint16_t* Uh = (uint16_t*)sm0;
    uint16_t* Ul = (uint16_t*)sm1;
    uint16_t* V = (uint16_t*)sm2;
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
    rank_update<MI, true>(acc, Uh, Ul, V, RP, l32, h, nc0, nc1);
    __syncthreads();
  }

  // global -> LDS streams (lane L of a direct load writes slot L): load q of wave w fills
  // rows (w*4+q)*16 .. +15 of its tile, lane L -> row + L/4, slot L%4 holding chunk
  // (L%4) ^ ((row >> 2) & 3).  Activation rows >= M read row M-1 and weight columns >=
  // out_f read column out_f-1 (their outputs are discarded).  The K-block advance is the
  // wave-uniform offset.
  constexpr int XQ = X_BYTES / 1024 / 4;
  constexpr int WQ = W_BYTES / 1024 / 4;
  constexpr int NLD = XQ + WQ;
  const rsrc_t xrs = make_rsrc(args.x + (size_t)m0 * K, (int64_t)(M - m0) * K * 2);
  uint32_t xoff[XQ];
#pragma unroll
  for (int q = 0; q < XQ; ++q) {
    const int row = (wave * XQ + q) * 16 + (lane >> 2);
    const int lr = (m0 + row < M) ? row : (M - 1 - m0);
    xoff[q] = 2u * ((uint32_t)lr * (uint32_t)K + (uint32_t)(((lane & 3) ^ ((row >> 2) & 3)) * 8));
  }
  const int64_t wbytes = (int64_t)out_f * K * 2;
  uint32_t woff[WQ];
#pragma unroll
  for (int q = 0; q < WQ; ++q) {
    const int col = (wave * WQ + q) * 16 + (lane >> 2);
    int n = nloc0 + col;
    n = n < out_f ? n : out_f - 1;
    woff[q] = (uint32_t)n * (uint32_t)K * 2u + (uint32_t)(((lane & 3) ^ ((col >> 2) & 3)) * 16);
  }
#define LNF4_FD_ISSUE_X(kb_, SM_)                                                                \
  {                                                                                              \
    const int kx_ = (kb_) < nk ? (kb_) : nk - 1;                                                 \
    _Pragma("unroll") for (int q = 0; q < XQ; ++q)                                               \
      LNF4_BUF_LDS(xrs, (SM_) + (wave_u * XQ + q) * 1024, 16, xoff[q], kx_ * (KS * 2));          \
  }
#define LNF4_FD_ISSUE_W(kb_, SM_)                                                                \
  {                                                                                              \
    const int kw_ = (kb_) < nk ? (kb_) : nk - 1;                                                 \
    const rsrc_t wrs_ = make_rsrc(P.w, (kb_) < nk ? wbytes : 0);                                 \
    _Pragma("unroll") for (int q = 0; q < WQ; ++q)                                               \
      LNF4_BUF_LDS(wrs_, (SM_) + X_BYTES + (wave_u * WQ + q) * 1024, 16, woff[q], kw_ * (KS * 2)); \
  }
  // fragments of step s: weight column col (MFMA A) and activation row block i (MFMA B)
#define LNF4_FD_WFRAG(SM_, s_, col_) \
  (*(const bf16x8*)((SM_) + X_BYTES + (col_) * 64 + ((((2 * h + (s_)) ^ (((col_) >> 2) & 3))) << 4)))
#define LNF4_FD_XFRAG(SM_, i_, s_)                                                               \
  (*(const bf16x8*)((SM_) + (32 * (i_) + l32) * 64 +                                             \
                    ((((2 * h + (s_)) ^ (((32 * (i_) + l32) >> 2) & 3))) << 4)))

  // prologue: blocks 0 .. 3 and the activation rows of block 4 in flight; block 0 visible
  LNF4_FD_ISSUE_X(0, sm0);
  LNF4_FD_ISSUE_W(0, sm0);
  LNF4_FD_ISSUE_X(1, sm1);
  LNF4_FD_ISSUE_W(1, sm1);
  LNF4_FD_ISSUE_X(2, sm2);
  LNF4_FD_ISSUE_W(2, sm2);
  LNF4_FD_ISSUE_X(3, sm3);
  LNF4_FD_ISSUE_W(3, sm3);
  LNF4_FD_ISSUE_X(4, sm4);
  LNF4_WAIT_VM(3 * NLD + XQ);
  __syncthreads();

  bf16x8 ac[MI], an_[MI];
  bf16x8 bc0, bc1, bn0, bn1;
  bc0 = LNF4_FD_WFRAG(sm0, 0, nc0);
  bc1 = LNF4_FD_WFRAG(sm0, 0, nc1);
#pragma unroll
  for (int i = 0; i < MI; ++i) ac[i] = LNF4_FD_XFRAG(sm0, i, 0);

  // One 32-wide block KB on stage SC; SN holds block KB+1, SP (the stage of KB-1) receives
  // the weight rows of block KB+4 at step 0.  Step 1: every wave's loads of block KB+1 have
  // landed (3 NLD loads issued after them may be in flight), the barrier makes KB+1 visible
  // and SC free, and the activation rows of block KB+5 go into SC.
#define LNF4_FD_BLOCK(KB, SC, SN, SP)                                                          \
  {                                                                                            \
    _Pragma("unroll") for (int s = 0; s < 2; ++s) {                                            \
      __builtin_amdgcn_sched_barrier(0);                                                       \
      if (s == 1) {                                                                            \
        LNF4_WAIT_VM_LGKM0(3 * NLD);                                                           \
        __builtin_amdgcn_s_barrier();                                                          \
        __builtin_amdgcn_sched_barrier(0);                                                     \
        bn0 = LNF4_FD_WFRAG(SN, 0, nc0);                                                       \
        bn1 = LNF4_FD_WFRAG(SN, 0, nc1);                                                       \
        _Pragma("unroll") for (int i = 0; i < MI; ++i) an_[i] = LNF4_FD_XFRAG(SN, i, 0);       \
        LNF4_FD_ISSUE_X((KB) + 5, SC);                                                         \
      } else {                                                                                 \
        bn0 = LNF4_FD_WFRAG(SC, 1, nc0);                                                       \
        bn1 = LNF4_FD_WFRAG(SC, 1, nc1);                                                       \
        _Pragma("unroll") for (int i = 0; i < MI; ++i) an_[i] = LNF4_FD_XFRAG(SC, i, 1);       \
        LNF4_FD_ISSUE_W((KB) + 4, SP);                                                         \
      }                                                                                        \
      _Pragma("unroll") for (int i = 0; i < MI; ++i) {                                         \
        acc[i][0] = mfma32(bc0, ac[i], acc[i][0]);                                             \
        acc[i][1] = mfma32(bc1, ac[i], acc[i][1]);                                             \
      }                                                                                        \
      _Pragma("unroll") for (int g = 0; g < NM; ++g) {                                         \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                     \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                     \
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                                     \
      }                                                                                        \
      _Pragma("unroll") for (int i = 0; i < MI; ++i) ac[i] = an_[i];                           \
      bc0 = bn0;                                                                               \
      bc1 = bn1;                                                                               \
    }                                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                         \
  }

  for (int kb = 0; kb < nk; kb += 5) {
    LNF4_FD_BLOCK(kb + 0, sm0, sm1, sm4);
    LNF4_FD_BLOCK(kb + 1, sm1, sm2, sm0);
    LNF4_FD_BLOCK(kb + 2, sm2, sm3, sm1);
    LNF4_FD_BLOCK(kb + 3, sm3, sm4, sm2);
    LNF4_FD_BLOCK(kb + 4, sm4, sm0, sm3);
  }
#undef LNF4_FD_BLOCK
#undef LNF4_FD_ISSUE_X
#undef LNF4_FD_ISSUE_W
#undef LNF4_FD_WFRAG
#undef LNF4_FD_XFRAG

  // ---- store bf16 (the 128-row kernel's scheme): lane (l32, h) has token 32i + l32 and,
  // for q = 4g..4g+3, the outputs 64 wave + 32j + 8g + 4h + 0..3.  With out_f % 8 == 0 and
  // y 16-byte aligned each wave stages its 256 rows in its own ring stage and stores whole
  // 128-byte lines; else 8-byte groups or single elements.
  if ((out_f & 7) == 0 && (((uintptr_t)P.y) & 15) == 0) {
    LNF4_WAIT_VM_LGKM0(0);  // the ring's last (past-the-end) loads have landed
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    uint8_t* const rg = wave == 0 ? sm0 : (wave == 1 ? sm1 : (wave == 2 ? sm2 : sm3));
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = 32 * i + l32;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int pc = (4 * j + g) ^ ((row >> 1) & 7);
          *(uint2*)(rg + row * 128 + pc * 16 + 8 * h) =
              make_uint2(pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                         pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]));
        }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging writes are done
    __builtin_amdgcn_sched_barrier(0);
    const int c = lane & 7;
    const int n = nloc0 + 64 * wave + 8 * c;
#pragma unroll
    for (int k = 0; k < BM / 8; ++k) {
      const int row = 8 * k + (lane >> 3);
      const u32x4 v = *(const u32x4*)(rg + row * 128 + ((c ^ ((row >> 1) & 7)) * 16));
      const int gm = m0 + row;
      if (gm < M && n < out_f) *(u32x4*)(P.y + (size_t)gm * out_f + n) = v;
    }
    return;
  }
  const bool vec4 = (out_f & 3) == 0 && (((uintptr_t)P.y) & 7) == 0;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    const int gm = m0 + 32 * i + l32;
    if (gm >= M) continue;
    uint16_t* yr = P.y + (size_t)gm * out_f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = nloc0 + 64 * wave + 32 * j + 8 * g + 4 * h;
        const float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        if (vec4 && n < out_f) {
          *(uint2*)(yr + n) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < out_f) yr[n + e] = __builtin_bit_cast(uint16_t, (__bf16)v[e]);
        }
      }
  }
}

// =====================================================================================
// Prefetch cursor over the K space of an input-gradient launch
// =====================================================================================
// The K-blocks a split loads run through the group's projections in order, so the
// projection that holds the next block to load (its pointers and out_f, read from the
// kernel arguments) changes at most n_proj - 1 times per split.  The cursor keeps that
// projection in scalar registers and otherwise only moves its row offset by one block.
// (Looking the projection up afresh for every block, a compare chain over the group and
// scalar loads of its fields with a wait on them, held up the wave's MFMA issue once per
// block.)  KS is the kernel's block height; the projections' kb0 count 64-row blocks.
struct DxCursor {
  int kb;    // next block to load
  int pi;    // its projection
  int next;  // first block of projection pi + 1 (INT_MAX after the last)
  int k0;    // its first row within the projection
  int Kp;    // the projection's out_f
  const uint16_t* dy;
  const void* w;
  const float* absmax;
};

template <int KS>
__device__ __forceinline__ void dx_cursor_load(DxCursor& c, const DxArgs& a) {
  const DxProj& P = a.p[c.pi];
  c.dy = P.dy;
  c.w = P.w;
  c.absmax = P.absmax;
  c.Kp = P.out_f;
  const int nx = c.pi + 1 < kMaxGroup ? c.pi + 1 : kMaxGroup - 1;
  c.next = c.pi + 1 < a.n_proj ? (64 / KS) * a.p[nx].kb0 : 0x7fffffff;
}

template <int KS>
__device__ __forceinline__ DxCursor dx_cursor_init(const DxArgs& a, int kb) {
  DxCursor c;
  int pi = 0;
#pragma unroll
  for (int q = 1; q < kMaxGroup; ++q)
    if (q < a.n_proj && kb >= (64 / KS) * a.p[q].kb0) pi = q;
  c.pi = __builtin_amdgcn_readfirstlane(pi);
  c.kb = kb;
  dx_cursor_load<KS>(c, a);
  c.k0 = (kb - (64 / KS) * a.p[c.pi].kb0) * KS;
  return c;
}

// move to the next block; true when it starts the next projection
template <int KS>
__device__ __forceinline__ bool dx_cursor_next(DxCursor& c, const DxArgs& a) {
  ++c.kb;
  c.k0 += KS;
  if (c.kb != c.next) return false;
  ++c.pi;
  dx_cursor_load<KS>(c, a);
  c.k0 = 0;
  return true;
}

// a byte count for a buffer resource, clamped to 2^31 - 1 with scalar operations
__device__ __forceinline__ int clamp31(uint64_t b) {
  return (uint32_t)(b >> 31) != 0u ? 0x7fffffff : (int)(uint32_t)b;
}

// =====================================================================================
// Input gradient, NF4 weights: direct-to-LDS ring with transposing code reads
// =====================================================================================
// dx [T][N] = sum over the group's K space (the projections' out rows) of dy . W'.
// The MFMA B operand needs 8 consecutive K (= 8 weight rows) of one column per lane, but
// the codes hold each row's columns contiguously.  The code tile [64 rows][256 cols] goes
// to LDS row-major by direct loads and is read back with ds_read_b64_tr_b4: in each group
// of 16 lanes, lane j names one 8-byte run (16 codes of one row) and lane i receives the
// i-th code of each of the 16 runs, i.e. 16 consecutive rows of one column.  With the
// high-nibble-first packing, code position i of a run is column i ^ 1, so lane l32 holds
// column l32 ^ 1 of its 32-column group; the accumulator columns follow that order.
// Each decoded value uses its own row's absmax (one fp32 product, one RNE, as in the
// forward).  absmax arrives as one 64-row column per wave ([wave][row], 4-byte loads).
template <int BM>
__global__ __launch_bounds__(NTHR, 1) void k_dxq(const DxArgs args) {
  constexpr int MI = BM / 32;
  constexpr int NM = 2 * MI;
  constexpr int X_BYTES = BM * BK * 2;     // dy tile [BM][64] bf16
  constexpr int W_BYTES = BK * BN / 2;     // codes [64][128 B]
  constexpr int A_BYTES = 4 * BK * 4;      // absmax [4 waves][64 rows] fp32
  constexpr int STAGE_RAW = X_BYTES + W_BYTES + A_BYTES;
  constexpr int SLAB_U = BM * LNF4_EPI_RANK * 2, SLAB_V = BN * LNF4_EPI_RANK * 2;
  constexpr int SLAB = SLAB_U > SLAB_V ? SLAB_U : SLAB_V;
  constexpr int STAGE = STAGE_RAW > SLAB ? STAGE_RAW : SLAB;
  // a 4-stage ring (blocks issued three ahead) where it fits LDS, else 3 stages
  constexpr int NSTG = 4 * STAGE + 2048 + 64 <= 160 * 1024 ? 4 : 3;
  static_assert(3 * STAGE + 2048 + 64 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint8_t sm0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm2[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm3[NSTG == 4 ? STAGE : 16];
  // byte-pair code table in transposed order: a byte of a transposed read holds rows 2b
  // (low nibble) and 2b+1 (high nibble) of one column; the large alignment places it at LDS
  // address 0, so an entry's address is just byte << 3
  __shared__ __attribute__((aligned(2048))) float2 lut2[256];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  lut2[tid] = make_float2(c_gemm_table[tid & 15], c_gemm_table[tid >> 4]);  // NTHR == 256

  int tm, tn;
  // split-K: workgroup b takes tile b % tiles and the split b / tiles of the K space
  const int n_tiles = args.n_tiles_m * args.n_tiles_n;
  const int split = (int)blockIdx.x / n_tiles;
  tile_coords((int)blockIdx.x - split * n_tiles, args.n_tiles_m, args.n_tiles_n, kGroupM, tm, tn);
  const int M = args.M, N = args.N;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb_beg = split * args.kb_per_split;
  const int kb_end = kb_beg + args.kb_per_split < args.total_kb ? kb_beg + args.kb_per_split : args.total_kb;
  // this lane's two accumulator columns within the tile (see the header comment)
  const int nc0 = 64 * wave + (l32 ^ 1), nc1 = nc0 + 32;

  // ---- accumulators start at the rank-R LoRA term (ranks of the group concatenated)
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
  if (R > 0 && split == 0) {  // the rank-R term once, in split 0
    const int RP = (R + 15) & ~15;
    uint16_t* Uh = (uint16_t*)sm0;
    uint16_t* Ul = (uint16_t*)sm1;
    uint16_t* V = (uint16_t*)sm2;
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
        if (gm < M) split_bf16(P.scale * P.v[(size_t)gm * P.v_stride + kk], Uh[mm * RP + off + kk], Ul[mm * RP + off + kk]);
      }
      for (int idx = tid; idx < BN * r; idx += NTHR) {
        const int kk = idx / BN, nn = idx - kk * BN, n = n0 + nn;
        if (n < N) V[nn * RP + off + kk] = P.A[(size_t)kk * N + n];
      }
      off += r;
    }
    __syncthreads();
    rank_update<MI, true>(acc, Uh, Ul, V, RP, l32, h, nc0, nc1);
    __syncthreads();
  }

  // ---- direct global -> LDS loads of one K-block (64 rows of one projection)
  //  * dy: load q of wave w fills tile rows (w*XQ+q)*8 .. +7 (as the forward's x)
  //  * codes: load q of wave w fills weight rows 16w+8q .. +7; lane L -> row 16w+8q+L/8,
  //    16-byte slot L%8 holding logical segment (L%8) ^ wswz(row)
  //  * absmax: one 4-byte load per wave, lane L -> row L of the wave's 64-column block
  //  Rows past the projection's out_f and columns past N read clamped addresses; their
  //  weights are zeroed by the decode (rows) or their outputs dropped (columns).
  constexpr int XQ = X_BYTES / 1024 / 4;
  static_assert(XQ % 2 == 0, "dy loads split over two steps");
  constexpr int NLD = XQ + 3;
  const int halfN = N / 2, nblk = N / 64;
  const int cbyte_max = halfN - 16;
  const int ablk = (n0 / 64 + wave) < nblk ? n0 / 64 + wave : nblk - 1;


  // per-lane constant parts of the buffer-load offsets (as in the forward kernels); the projection and the
  // K offset go into each block's resources, whose ranges end at the projection's last
  // row, so rows past out_f load as zeros: zero absmax, hence zero weights
  uint32_t dyr2[XQ], dyc[XQ];
#pragma unroll
  for (int q = 0; q < XQ; ++q) {
    const int row = (wave * XQ + q) * 8 + (lane >> 3);
    dyr2[q] = 2u * (uint32_t)(m0 + row < M ? m0 + row : M - 1);
    dyc[q] = 16u * (uint32_t)((lane & 7) ^ act_swz(row));
  }
  uint32_t cwoff[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = 16 * wave + 8 * q + (lane >> 3);
    const int cb = n0 / 2 + 16 * ((lane & 7) ^ wswz(row));
    cwoff[q] = (uint32_t)row * (uint32_t)halfN + (uint32_t)(cb < cbyte_max ? cb : cbyte_max);
  }
  const uint32_t caoff = 4u * ((uint32_t)lane * (uint32_t)nblk + (uint32_t)ablk);

  // The loads of one K-block go out in three parts, one per step of the block before the
  // ring wraps: dy rows of the first half, of the second half, then codes and absmax.
  // The block is the prefetch cursor's; its resources end at the projection's last row.
  // Blocks past the split (the loop runs whole trips) get empty resources, and every load
  // returns zeros (zero dy, zero absmax).  Branch-free: a branch would split the step.
  DxCursor cur = dx_cursor_init<BK>(args, kb_beg);
  uint32_t dyo[XQ];
#pragma unroll
  for (int q = 0; q < XQ; ++q) dyo[q] = dyr2[q] * (uint32_t)cur.Kp + dyc[q];
#define LNF4_DXQ_RSRC()                                                                          \
    const int live_ = -(int)((cur.kb < kb_end) & (cur.k0 < cur.Kp));                             \
    const uint32_t rows_ = (uint32_t)((cur.Kp - cur.k0) & live_);                                \
    const rsrc_t dyrs_ = make_rsrc_n(                                                            \
        cur.dy + cur.k0, clamp31(((uint64_t)(uint32_t)M * (uint32_t)cur.Kp - (uint32_t)cur.k0) * 2u) & live_); \
    const rsrc_t wrs_ = make_rsrc_n((const uint8_t*)cur.w + (size_t)cur.k0 * halfN,               \
                                    clamp31((uint64_t)rows_ * (uint32_t)halfN));                  \
    const rsrc_t ars_ = make_rsrc_n(cur.absmax + (size_t)cur.k0 * nblk,                          \
                                    clamp31((uint64_t)rows_ * (uint32_t)(4 * nblk)));
  // the cursor moves after the block's last step, outside its interleaved regions
#define LNF4_DXQ_ADVANCE()                                                                       \
  {                                                                                              \
    if (dx_cursor_next<BK>(cur, args)) {                                                         \
      _Pragma("unroll") for (int q = 0; q < XQ; ++q) dyo[q] = dyr2[q] * (uint32_t)cur.Kp + dyc[q]; \
    }                                                                                            \
  }
#define LNF4_DXQ_ISSUE_PART(SM_, part_)                                                          \
  {                                                                                              \
    if ((part_) < 2) {                                                                           \
      _Pragma("unroll") for (int q = (part_) * (XQ / 2); q < ((part_) + 1) * (XQ / 2); ++q)      \
          LNF4_BUF_LDS(dyrs_, (SM_) + (wave_u * XQ + q) * 1024, 16, dyo[q], 0);                 \
    } else {                                                                                     \
      _Pragma("unroll") for (int q = 0; q < 2; ++q)                                              \
          LNF4_BUF_LDS(wrs_, (SM_) + X_BYTES + (wave_u * 2 + q) * 1024, 16, cwoff[q], 0);        \
      LNF4_BUF_LDS(ars_, (SM_) + X_BYTES + W_BYTES + wave_u * 256, 4, caoff, 0);                  \
    }                                                                                            \
  }
#define LNF4_DXQ_ISSUE(SM_)                                                                      \
  {                                                                                              \
    LNF4_DXQ_RSRC()                                                                              \
    LNF4_DXQ_ISSUE_PART(SM_, 0)                                                                  \
    LNF4_DXQ_ISSUE_PART(SM_, 1)                                                                  \
    LNF4_DXQ_ISSUE_PART(SM_, 2)                                                                  \
  }                                                                                              \
  LNF4_DXQ_ADVANCE()

  typedef int v2i_t __attribute__((ext_vector_type(2)));
  // transposed code reads of one stage: cw[s] = 8 codes (rows 32h+8s .. +7) of the column
  const int trow0 = 32 * h + (lane & 15), trow1 = trow0 + 16;
  const int tpart = 8 * ((lane >> 4) & 1);
  const int toff00 = trow0 * 128 + 16 * ((2 * wave + 0) ^ wswz(trow0)) + tpart;
  const int toff01 = trow1 * 128 + 16 * ((2 * wave + 0) ^ wswz(trow1)) + tpart;
  const int toff10 = trow0 * 128 + 16 * ((2 * wave + 1) ^ wswz(trow0)) + tpart;
  const int toff11 = trow1 * 128 + 16 * ((2 * wave + 1) ^ wswz(trow1)) + tpart;
#define LNF4_TR4(SM_, off_) \
  __builtin_amdgcn_ds_read_tr4_b64_v2i32((__attribute__((address_space(3))) v2i_t*)((SM_) + X_BYTES + (off_)))
#define LNF4_DXQ_CODES(SM_, c0_, c1_)                              \
  {                                                                \
    const v2i_t a_ = LNF4_TR4(SM_, toff00), b_ = LNF4_TR4(SM_, toff01); \
    const v2i_t c_ = LNF4_TR4(SM_, toff10), d_ = LNF4_TR4(SM_, toff11); \
    c0_ = u32x4{(uint32_t)a_.x, (uint32_t)a_.y, (uint32_t)b_.x, (uint32_t)b_.y}; \
    c1_ = u32x4{(uint32_t)c_.x, (uint32_t)c_.y, (uint32_t)d_.x, (uint32_t)d_.y}; \
  }
  // absmax of rows 32h+8s .. +7 of this wave's column block
#define LNF4_DXQ_SCALES(SM_, s_, a_)                                                              \
  {                                                                                              \
    const float* ap_ = (const float*)((SM_) + X_BYTES + W_BYTES + wave * 256) + 32 * h + 8 * (s_); \
    const floatx4 lo_ = *(const floatx4*)ap_, hi_ = *(const floatx4*)(ap_ + 4);                  \
    a_[0] = lo_[0]; a_[1] = lo_[1]; a_[2] = lo_[2]; a_[3] = lo_[3];                             \
    a_[4] = hi_[0]; a_[5] = hi_[1]; a_[6] = hi_[2]; a_[7] = hi_[3];                             \
  }
#define LNF4_LUT8X(lv, cw_)                                                        \
  {                                                                                \
    const uint32_t c_ = (cw_);                                                     \
    _Pragma("unroll") for (int b_ = 0; b_ < 4; ++b_) {                             \
      const float2 p_ = lut2[(c_ >> (8 * b_)) & 255u];                             \
      lv[2 * b_] = p_.x;                                                           \
      lv[2 * b_ + 1] = p_.y;                                                       \
    }                                                                              \
  }
#define LNF4_FIN8X(dst, lv, a_)                                                    \
  dst = as_bf16x8(pack_bf16x2(lv[0] * a_[0], lv[1] * a_[1]), pack_bf16x2(lv[2] * a_[2], lv[3] * a_[3]), \
                  pack_bf16x2(lv[4] * a_[4], lv[5] * a_[5]), pack_bf16x2(lv[6] * a_[6], lv[7] * a_[7]));
#define LNF4_XS(SM_) ((const uint16_t*)(SM_))

  // prologue: blocks 0 .. NSTG-2 in flight; block 0 visible
  LNF4_DXQ_ISSUE(sm0);
  LNF4_DXQ_ISSUE(sm1);
  if (NSTG == 4) { LNF4_DXQ_ISSUE(sm2); }
  LNF4_WAIT_VM((NSTG - 2) * NLD);
  __syncthreads();

  bf16x8 ac[MI], an_[MI];
  bf16x8 bc0, bc1, bn0, bn1;
  u32x4 cw0, cw1;
  {
    LNF4_DXQ_CODES(sm0, cw0, cw1);
    float l0[8], l1[8], a[8];
    LNF4_LUT8X(l0, cw0[0]);
    LNF4_LUT8X(l1, cw1[0]);
    LNF4_DXQ_SCALES(sm0, 0, a);
    LNF4_FIN8X(bc0, l0, a);
    LNF4_FIN8X(bc1, l1, a);
  }
#pragma unroll
  for (int i = 0; i < MI; ++i) ac[i] = *(const bf16x8*)&LNF4_XS(sm0)[act_pos(32 * i + l32, 4 * h)];

  // One K-block KB on stage SC; SN holds block KB+1, SP receives block KB+NSTG-1 (issued in
  // parts over steps 0..2, each after the step's LDS reads).
#define LNF4_DXQ_BLOCK(KB, SC, SN, SP)                                                         \
  {                                                                                            \
    u32x4 nw0, nw1;                                                                            \
    LNF4_DXQ_RSRC()                                                                            \
    _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                            \
      __builtin_amdgcn_sched_barrier(0);                                                       \
      if (s == 3) {                                                                            \
        /* block KB+1 in LDS for every wave; every wave done with SC */                        \
        LNF4_WAIT_VM_LGKM0((NSTG - 2) * NLD);                                                  \
        __builtin_amdgcn_s_barrier();                                                          \
        __builtin_amdgcn_sched_barrier(0);                                                     \
      }                                                                                        \
      float l0[8], l1[8], a[8];                                                                \
      if (s < 3) {                                                                             \
        LNF4_LUT8X(l0, cw0[s + 1 < 4 ? s + 1 : 0]);                                            \
        LNF4_LUT8X(l1, cw1[s + 1 < 4 ? s + 1 : 0]);                                            \
        LNF4_DXQ_SCALES(SC, (s + 1 < 4 ? s + 1 : 0), a);                                       \
      } else {                                                                                 \
        LNF4_DXQ_CODES(SN, nw0, nw1);                                                          \
        LNF4_LUT8X(l0, nw0[0]);                                                                \
        LNF4_LUT8X(l1, nw1[0]);                                                                \
        LNF4_DXQ_SCALES(SN, 0, a);                                                             \
      }                                                                                        \
      if (s < 3) {                                                                             \
        _Pragma("unroll") for (int i = 0; i < MI; ++i) an_[i] =                                \
            *(const bf16x8*)&LNF4_XS(SC)[act_pos(32 * i + l32, 4 * h + s + 1)];                \
      } else {                                                                                 \
        _Pragma("unroll") for (int i = 0; i < MI; ++i) an_[i] =                                \
            *(const bf16x8*)&LNF4_XS(SN)[act_pos(32 * i + l32, 4 * h)];                        \
      }                                                                                        \
      if (s < 3) LNF4_DXQ_ISSUE_PART(SP, s);                                                   \
      _Pragma("unroll") for (int i = 0; i < MI; ++i) {                                         \
        acc[i][0] = mfma32(bc0, ac[i], acc[i][0]);                                             \
        acc[i][1] = mfma32(bc1, ac[i], acc[i][1]);                                             \
      }                                                                                        \
      LNF4_FIN8X(bn0, l0, a);                                                                  \
      LNF4_FIN8X(bn1, l1, a);                                                                  \
      _Pragma("unroll") for (int g = 0; g < 4; ++g) {                                          \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                     \
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);                                     \
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);                                     \
      }                                                                                        \
      _Pragma("unroll") for (int g = 4; g < NM - NM / 4; ++g) {                                \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                     \
        __builtin_amdgcn_sched_group_barrier(0x100, (MI + (NM - NM / 4 - 4) - 1) / (NM - NM / 4 - 4), 0); \
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                                     \
      }                                                                                        \
      _Pragma("unroll") for (int g = NM - NM / 4; g < NM; ++g) {                               \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                     \
        __builtin_amdgcn_sched_group_barrier(0x002, (32 + NM / 4 - 1) / (NM / 4), 0);          \
      }                                                                                        \
      _Pragma("unroll") for (int i = 0; i < MI; ++i) ac[i] = an_[i];                           \
      bc0 = bn0;                                                                               \
      bc1 = bn1;                                                                               \
    }                                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                         \
    asm volatile("" ::"v"(bc0), "v"(bc1)); /* decoded before the exit test */            \
    cw0 = nw0;                                                                                 \
    cw1 = nw1;                                                                                 \
    LNF4_DXQ_ADVANCE();                                                                        \
  }

  // whole trips of two turns of the ring, one exit test per trip (blocks past the last
  // add zeros)
  if constexpr (NSTG == 4) {
    for (int kb = kb_beg; kb < kb_end; kb += 8) {
      LNF4_DXQ_BLOCK(kb + 0, sm0, sm1, sm3);
      LNF4_DXQ_BLOCK(kb + 1, sm1, sm2, sm0);
      LNF4_DXQ_BLOCK(kb + 2, sm2, sm3, sm1);
      LNF4_DXQ_BLOCK(kb + 3, sm3, sm0, sm2);
      LNF4_DXQ_BLOCK(kb + 4, sm0, sm1, sm3);
      LNF4_DXQ_BLOCK(kb + 5, sm1, sm2, sm0);
      LNF4_DXQ_BLOCK(kb + 6, sm2, sm3, sm1);
      LNF4_DXQ_BLOCK(kb + 7, sm3, sm0, sm2);
    }
  } else {
    for (int kb = kb_beg; kb < kb_end; kb += 6) {
      LNF4_DXQ_BLOCK(kb + 0, sm0, sm1, sm2);
      LNF4_DXQ_BLOCK(kb + 1, sm1, sm2, sm0);
      LNF4_DXQ_BLOCK(kb + 2, sm2, sm0, sm1);
      LNF4_DXQ_BLOCK(kb + 3, sm0, sm1, sm2);
      LNF4_DXQ_BLOCK(kb + 4, sm1, sm2, sm0);
      LNF4_DXQ_BLOCK(kb + 5, sm2, sm0, sm1);
    }
  }
#undef LNF4_DXQ_BLOCK
#undef LNF4_DXQ_ADVANCE
#undef LNF4_DXQ_ISSUE
#undef LNF4_DXQ_ISSUE_PART
#undef LNF4_DXQ_RSRC
#undef LNF4_TR4
#undef LNF4_DXQ_CODES
#undef LNF4_DXQ_SCALES
#undef LNF4_LUT8X
#undef LNF4_FIN8X
#undef LNF4_XS

  // ---- store.  The decoded weights are the MFMA's A operand, so the accumulators hold the
  // tile transposed: lane (l32, h) has token 32i + l32 and, for q = 4g..4g+3, accumulator
  // rows 8g + 4h + 0..3, i.e. tile columns 64 wave + 32j + 8g + 4h + (e ^ 1) for e = 0..3
  // (a lane's weight column is l32 ^ 1, see the header comment).  Rows go out through LDS
  // in passes of 64: each wave stages its 64 columns of them as fp32 (16-byte chunk c of row
  // r at c ^ (r & 15)) and reads back whole rows, 16 lanes per row, so every store covers
  // full 128-byte lines of the output.  fp32 staging keeps one rounding when accumulating.
  const int n_w = n0 + 64 * wave;
  float* const pp = args.part != nullptr ? args.part + (size_t)split * M * N : nullptr;
  if (pp != nullptr || (((uintptr_t)args.dx) & 7) == 0) {
    LNF4_WAIT_VM_LGKM0(0);  // the ring's last (past-the-end) loads have landed
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    uint8_t* const rg = (wave < 2 ? sm0 : sm1) + (wave & 1) * 16384;
#pragma unroll
    for (int pass = 0; pass < MI / 2; ++pass) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * pass + ii, row = 32 * ii + l32;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int pc = (8 * j + 2 * g + h) ^ (row & 15);
            floatx4 v;
            v[0] = acc[i][j][4 * g + 1];
            v[1] = acc[i][j][4 * g];
            v[2] = acc[i][j][4 * g + 3];
            v[3] = acc[i][j][4 * g + 2];
            *(floatx4*)(rg + row * 256 + pc * 16) = v;
          }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging writes are done
      __builtin_amdgcn_sched_barrier(0);
      const int c = lane & 15, n = n_w + 4 * c;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int row = 4 * k + (lane >> 4);
        floatx4 v = *(const floatx4*)(rg + row * 256 + ((c ^ (row & 15)) * 16));
        const int gm = m0 + 64 * pass + row;
        if (gm >= M || n >= N) continue;
        if (pp != nullptr) {
          *(floatx4*)(pp + (size_t)gm * N + n) = v;
        } else {
          uint16_t* d = args.dx + (size_t)gm * N + n;
          if (args.accumulate) {
            const uint2 o = *(const uint2*)d;
            v[0] += bf16_lo(o.x); v[1] += bf16_hi(o.x); v[2] += bf16_lo(o.y); v[3] += bf16_hi(o.y);
          }
          *(uint2*)d = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }
  // dx only 2-byte aligned: element by element
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    const int gm = m0 + 32 * i + l32;
    if (gm >= M) continue;
    uint16_t* dr = args.dx + (size_t)gm * N;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int n = n_w + 32 * j + 8 * (q >> 2) + 4 * h + ((q & 3) ^ 1);
        if (n >= N) continue;
        float v = acc[i][j][q];
        if (args.accumulate) v += bf16_to_f32(dr[n]);
        dr[n] = __builtin_bit_cast(uint16_t, (__bf16)v);
      }
  }
}

// Rank-R LoRA term of the bf16-weight input gradient (ranks of the group concatenated),
// folded into the accumulators: hi and lo halves of s_p v_p staged in Uh / Ul [BM][RP],
// the adapter columns of the tile in V [256][RP] (three LDS slabs of BM x 64 and 256 x 64
// bf16), then the rank update on the MFMA units.  Accumulators are not transposed.
template <int MI>
__device__ __forceinline__ void dx_bf16_rank_init(floatx16 (&acc)[MI][2], const DxArgs& args, int m0, int n0,
                                                  uint8_t* s_uh, uint8_t* s_ul, uint8_t* s_v, int tid, int l32,
                                                  int h, int nc0, int nc1) {
  constexpr int BM = 32 * MI;
  const int M = args.M, N = args.N;
  int R = 0;
  for (int pi = 0; pi < args.n_proj; ++pi) {
    const DxProj P = select_dx(args, pi);
    if (P.v != nullptr && P.r > 0) R += P.r;
  }
  if (R <= 0) return;
  const int RP = (R + 15) & ~15;
  uint16_t* Uh = (uint16_t*)s_uh;
  uint16_t* Ul = (uint16_t*)s_ul;
  uint16_t* V = (uint16_t*)s_v;
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
      if (gm < M) split_bf16(P.scale * P.v[(size_t)gm * P.v_stride + kk], Uh[mm * RP + off + kk], Ul[mm * RP + off + kk]);
    }
    for (int idx = tid; idx < BN * r; idx += NTHR) {
      const int kk = idx / BN, nn = idx - kk * BN, n = n0 + nn;
      if (n < N) V[nn * RP + off + kk] = P.A[(size_t)kk * N + n];
    }
    off += r;
  }
  __syncthreads();
  rank_update<MI>(acc, Uh, Ul, V, RP, l32, h, nc0, nc1);
  __syncthreads();
}

// Output of a bf16-weight input-gradient tile: this split's fp32 sums into the split-K
// workspace, or bf16 dx (optionally added to the existing dx).  Lane (l32, h) holds columns
// nc0 / nc1 and, for q = 0..15, row 32i + 8(q / 4) + 4h + q % 4 of the tile.
template <int MI>
__device__ __forceinline__ void dx_bf16_store(const floatx16 (&acc)[MI][2], const DxArgs& args, int split, int m0,
                                              int n0, int nc0, int nc1, int h) {
  const int M = args.M, N = args.N;
  const int n0g = n0 + nc0, n1g = n0 + nc1;
  const bool c0ok = n0g < N, c1ok = n1g < N;
  if (args.part != nullptr) {  // split-K: this split's fp32 sums, added up by k_dx_split_sum
    float* pp = args.part + (size_t)split * M * N;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int gm = m0 + 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);
        if (gm >= M) continue;
        if (c0ok) pp[(size_t)gm * N + n0g] = acc[i][0][q];
        if (c1ok) pp[(size_t)gm * N + n1g] = acc[i][1][q];
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int gm = m0 + 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);
      if (gm >= M) continue;
      uint16_t* dr = args.dx + (size_t)gm * N;
      float v0 = acc[i][0][q], v1 = acc[i][1][q];
      if (args.accumulate) {
        if (c0ok) v0 += bf16_to_f32(dr[n0g]);
        if (c1ok) v1 += bf16_to_f32(dr[n1g]);
      }
      if (c0ok) dr[n0g] = __builtin_bit_cast(uint16_t, (__bf16)v0);
      if (c1ok) dr[n1g] = __builtin_bit_cast(uint16_t, (__bf16)v1);
    }
  }
}


// =====================================================================================
// Input gradient, bf16 weights: direct-to-LDS ring with transposing 16-bit reads
// =====================================================================================
// dx [T][N] = sum over the group's K space of dy . W' with W' bf16 [K rows][N], N
// contiguous.  The weight tile [64 rows][256 cols] goes to LDS row-major by direct loads
// (512-byte rows of 32 16-byte chunks, chunk c of row r stored at c ^ 4(r & 3)) and is read
// back with ds_read_b64_tr_b16: in each group of 16 lanes, lane a + 4c names the 4-column
// run (4a .. 4a+3) of row k0 + c, and lane i of the group receives column i of those four
// rows.  Two such reads give a lane the 8 consecutive K of one column that the MFMA B
// operand takes (in the activation tile's K order); the four rows of one read then cover
// all 16 chunk banks, so a read takes the minimum two LDS cycles.
template <int BM>
__global__ __launch_bounds__(NTHR, 1) void k_dx_bf16(const DxArgs args) {
  constexpr int MI = BM / 32;
  constexpr int NM = 2 * MI;
  constexpr int X_BYTES = BM * BK * 2;     // dy tile [BM][64] bf16
  constexpr int W_BYTES = BK * BN * 2;     // weight tile [64][256] bf16
  constexpr int STAGE_RAW = X_BYTES + W_BYTES;
  constexpr int SLAB_U = BM * LNF4_EPI_RANK * 2, SLAB_V = BN * LNF4_EPI_RANK * 2;
  constexpr int SLAB = SLAB_U > SLAB_V ? SLAB_U : SLAB_V;
  constexpr int STAGE = STAGE_RAW > SLAB ? STAGE_RAW : SLAB;
  static_assert(3 * STAGE <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint8_t sm0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm2[STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  int tm, tn;
  // split-K: workgroup b takes tile b % tiles and the split b / tiles of the K space
  const int n_tiles = args.n_tiles_m * args.n_tiles_n;
  const int split = (int)blockIdx.x / n_tiles;
  tile_coords((int)blockIdx.x - split * n_tiles, args.n_tiles_m, args.n_tiles_n, kGroupM, tm, tn);
  const int M = args.M, N = args.N;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kb_beg = split * args.kb_per_split;
  const int kb_end = kb_beg + args.kb_per_split < args.total_kb ? kb_beg + args.kb_per_split : args.total_kb;
  const int nc0 = 64 * wave + l32, nc1 = nc0 + 32;

  // ---- accumulators start at the rank-R LoRA term (ranks of the group concatenated)
  floatx16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  if (split == 0) dx_bf16_rank_init<MI>(acc, args, m0, n0, sm0, sm1, sm2, tid, l32, h, nc0, nc1);

  // ---- direct global -> LDS loads of one K-block (64 rows of one projection)
  //  * dy: load q of wave w fills tile rows (w*XQ+q)*8 .. +7 (as the forward's x)
  //  * weights: load q of wave w fills rows 2g, 2g+1 (g = w*WQ+q); lane L -> row 2g + L/32,
  //    stored chunk L%32, which holds global chunk (L%32) ^ 4(row & 3) of the row
  //  Rows past the projection's out_f load zeros (the block's resources end there);
  //  columns past N belong to outputs that are dropped.
  constexpr int XQ = X_BYTES / 1024 / 4;
  constexpr int WQ = W_BYTES / 1024 / 4;
  constexpr int NLD = XQ + WQ;
  static_assert(NLD % 3 == 0, "loads split over three steps");
  uint32_t dyr2[XQ], dyc[XQ];
#pragma unroll
  for (int q = 0; q < XQ; ++q) {
    const int row = (wave * XQ + q) * 8 + (lane >> 3);
    dyr2[q] = 2u * (uint32_t)(m0 + row < M ? m0 + row : M - 1);
    dyc[q] = 16u * (uint32_t)((lane & 7) ^ act_swz(row));
  }
  uint32_t woff[WQ];
#pragma unroll
  for (int q = 0; q < WQ; ++q) {
    const int row = 2 * (wave * WQ + q) + (lane >> 5);
    const int cg = (lane & 31) ^ (4 * (row & 3));
    woff[q] = 2u * ((uint32_t)row * (uint32_t)N + (uint32_t)(n0 + 8 * cg));
  }

  // The block is the prefetch cursor's; its resources end at the projection's last row
  // (rows past out_f load zeros).  Blocks past the split (the loop runs whole trips) get
  // empty resources and every load returns zeros.  Branch-free: a branch would split the
  // step.
  DxCursor cur = dx_cursor_init<BK>(args, kb_beg);
  uint32_t dyo[XQ];
#pragma unroll
  for (int q = 0; q < XQ; ++q) dyo[q] = dyr2[q] * (uint32_t)cur.Kp + dyc[q];
#define LNF4_DXB_RSRC()                                                                          \
    const int live_ = -(int)((cur.kb < kb_end) & (cur.k0 < cur.Kp));                             \
    const rsrc_t dyrs_ = make_rsrc_n(                                                            \
        cur.dy + cur.k0, clamp31(((uint64_t)(uint32_t)M * (uint32_t)cur.Kp - (uint32_t)cur.k0) * 2u) & live_); \
    const rsrc_t wrs_ = make_rsrc_n((const uint16_t*)cur.w + (size_t)cur.k0 * N,                 \
        clamp31((uint64_t)(uint32_t)((cur.Kp - cur.k0) & live_) * (2u * (uint32_t)N)));
  // the cursor moves after the block's last step, outside its interleaved regions
#define LNF4_DXB_ADVANCE()                                                                       \
  {                                                                                              \
    if (dx_cursor_next<BK>(cur, args)) {                                                         \
      _Pragma("unroll") for (int q = 0; q < XQ; ++q) dyo[q] = dyr2[q] * (uint32_t)cur.Kp + dyc[q]; \
    }                                                                                            \
  }
  // load i of a block (0 .. NLD-1): dy loads first, then weight loads
#define LNF4_DXB_LOAD1(SM_, i_)                                                                  \
  {                                                                                              \
    if ((i_) < XQ)                                                                               \
      LNF4_BUF_LDS(dyrs_, (SM_) + (wave_u * XQ + (i_)) * 1024, 16, dyo[(i_) < XQ ? (i_) : 0], 0); \
    else                                                                                         \
      LNF4_BUF_LDS(wrs_, (SM_) + X_BYTES + (wave_u * WQ + (i_) - XQ) * 1024, 16, woff[(i_) < XQ ? 0 : (i_) - XQ], 0); \
  }
#define LNF4_DXB_ISSUE_PART(SM_, part_)                                                          \
  { _Pragma("unroll") for (int i = (part_) * (NLD / 3); i < ((part_) + 1) * (NLD / 3); ++i) LNF4_DXB_LOAD1(SM_, i) }
#define LNF4_DXB_ISSUE(SM_)                                                                      \
  {                                                                                              \
    LNF4_DXB_RSRC()                                                                              \
    LNF4_DXB_ISSUE_PART(SM_, 0)                                                                  \
    LNF4_DXB_ISSUE_PART(SM_, 1)                                                                  \
    LNF4_DXB_ISSUE_PART(SM_, 2)                                                                  \
  }                                                                                              \
  LNF4_DXB_ADVANCE()

  typedef short v4s_t __attribute__((ext_vector_type(4)));
  // transposing reads: lane j = a + 4c of its 16-lane group (j = lane % 16) names row
  // base + c, columns 16g + 4a .. +3 of its 32-column block (g = l32 / 16)
  const int tr_c = (lane & 15) >> 2, tr_col = 16 * ((lane & 31) >> 4) + 4 * (lane & 3);
  // byte offset of the run for row `row` (row & 3 == tr_c) and column `col`
#define LNF4_TRB(SM_, row_, col_)                                                                \
  __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(           \
      (SM_) + X_BYTES + (row_) * 512 + ((((col_) >> 3) ^ (4 * ((row_) & 3))) << 4) + (((col_) & 7) << 1)))
  // B fragment of step s (K = 32h + 8s .. +7) for the 32-column block starting at cb
  const int tbo0 = (32 * h + tr_c) * 512 + (((8 * wave + 0 + (tr_col >> 3)) ^ (4 * tr_c)) << 4) + ((tr_col & 7) << 1);
  const int tbo1 = (32 * h + tr_c) * 512 + (((8 * wave + 4 + (tr_col >> 3)) ^ (4 * tr_c)) << 4) + ((tr_col & 7) << 1);
#define LNF4_TRO(SM_, off_) \
  __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)((SM_) + X_BYTES + (off_)))
#define LNF4_DXB_FRAG(SM_, s_, cb_)                                                              \
  ({                                                                                             \
    const int o_ = ((cb_) == 64 * wave ? tbo0 : tbo1) + 4096 * (s_);                              \
    const v4s_t lo_ = LNF4_TRO(SM_, o_);                                                         \
    const v4s_t hi_ = LNF4_TRO(SM_, o_ + 2048);                                                  \
    __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo_, hi_, 0, 1, 2, 3, 4, 5, 6, 7));      \
  })
#define LNF4_XS(SM_) ((const uint16_t*)(SM_))

  // prologue: blocks 0 and 1 in flight; block 0 visible
  LNF4_DXB_ISSUE(sm0);
  LNF4_DXB_ISSUE(sm1);
  LNF4_WAIT_VM(NLD);
  __syncthreads();

  bf16x8 ac[MI], an_[MI];
  bf16x8 bc0, bc1, bn0, bn1;
  bc0 = LNF4_DXB_FRAG(sm0, 0, 64 * wave);
  bc1 = LNF4_DXB_FRAG(sm0, 0, 64 * wave + 32);
#pragma unroll
  for (int i = 0; i < MI; ++i) ac[i] = *(const bf16x8*)&LNF4_XS(sm0)[act_pos(32 * i + l32, 4 * h)];

  // One K-block KB on stage SC; SN holds block KB+1, SP receives block KB+2 (issued in
  // parts over steps 0..2, each after the step's LDS reads).
#define LNF4_DXB_BLOCK(KB, SC, SN, SP)                                                         \
  {                                                                                            \
    LNF4_DXB_RSRC()                                                                            \
    _Pragma("unroll") for (int s = 0; s < 4; ++s) {                                            \
      __builtin_amdgcn_sched_barrier(0);                                                       \
      if (s == 3) {                                                                            \
        /* block KB+1 in LDS for every wave; every wave done with SC */                        \
        LNF4_WAIT_VM_LGKM0(NLD);                                                               \
        __builtin_amdgcn_s_barrier();                                                          \
        __builtin_amdgcn_sched_barrier(0);                                                     \
      }                                                                                        \
      if (s < 3) {                                                                             \
        bn0 = LNF4_DXB_FRAG(SC, s + 1, 64 * wave);                                             \
        bn1 = LNF4_DXB_FRAG(SC, s + 1, 64 * wave + 32);                                        \
        _Pragma("unroll") for (int i = 0; i < MI; ++i) an_[i] =                                \
            *(const bf16x8*)&LNF4_XS(SC)[act_pos(32 * i + l32, 4 * h + s + 1)];                \
      } else {                                                                                 \
        bn0 = LNF4_DXB_FRAG(SN, 0, 64 * wave);                                                 \
        bn1 = LNF4_DXB_FRAG(SN, 0, 64 * wave + 32);                                            \
        _Pragma("unroll") for (int i = 0; i < MI; ++i) an_[i] =                                \
            *(const bf16x8*)&LNF4_XS(SN)[act_pos(32 * i + l32, 4 * h)];                        \
      }                                                                                        \
      if (s < 3) LNF4_DXB_ISSUE_PART(SP, s);                                                   \
      _Pragma("unroll") for (int i = 0; i < MI; ++i) {                                         \
        acc[i][0] = mfma32(ac[i], bc0, acc[i][0]);                                             \
        acc[i][1] = mfma32(ac[i], bc1, acc[i][1]);                                             \
      }                                                                                        \
      _Pragma("unroll") for (int g = 0; g < NM; ++g) {                                         \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                     \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                     \
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                                     \
      }                                                                                        \
      _Pragma("unroll") for (int i = 0; i < MI; ++i) ac[i] = an_[i];                           \
      bc0 = bn0;                                                                               \
      bc1 = bn1;                                                                               \
    }                                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                         \
    LNF4_DXB_ADVANCE();                                                                        \
  }

  // whole trips of two turns of the 3-stage ring, one exit test per trip (blocks past the
  // last add zeros)
  for (int kb = kb_beg; kb < kb_end; kb += 6) {
    LNF4_DXB_BLOCK(kb + 0, sm0, sm1, sm2);
    LNF4_DXB_BLOCK(kb + 1, sm1, sm2, sm0);
    LNF4_DXB_BLOCK(kb + 2, sm2, sm0, sm1);
    LNF4_DXB_BLOCK(kb + 3, sm0, sm1, sm2);
    LNF4_DXB_BLOCK(kb + 4, sm1, sm2, sm0);
    LNF4_DXB_BLOCK(kb + 5, sm2, sm0, sm1);
  }
#undef LNF4_DXB_BLOCK
#undef LNF4_DXB_ADVANCE
#undef LNF4_DXB_RSRC
#undef LNF4_DXB_LOAD1
#undef LNF4_DXB_ISSUE_PART
#undef LNF4_DXB_ISSUE
#undef LNF4_TRB
#undef LNF4_DXB_FRAG
#undef LNF4_XS

  dx_bf16_store<MI>(acc, args, split, m0, n0, nc0, nc1, h);
}

// Input gradient, bf16 weights, 256-row tiles: 32-wide K-blocks in a 5-stage ring.
// A 256 x 256 tile loads 32 KB per 32 K (dy [256][32] and W [32][256]), 1.5x fewer bytes per
// MFMA than the 128-row tile, but with 64-wide blocks only two 64 KB stages fit LDS and a
// block's loads then have one block of MFMAs (about 2,000 cycles) to land, less than the
// latency of the streamed operands of a long-K launch such as the lm_head input gradient.
// With 32-wide blocks five 32 KB stages fit (160 KB): a block's loads are issued right
// after the barrier that frees its stage, four blocks (128 MFMAs per wave) before they are
// read.
//  * K order inside a block: lane (n, h) of the MFMA supplies K = 16h + 8s .. +7 at step s
//    (two steps per block); the dy tile's 64-byte rows hold four 16-byte chunks, chunk c of
//    row r at slot c ^ ((r >> 2) & 3), so the 16 rows one read phase serves cover all 16
//    bank groups.
//  * Weight rows (K) are 512 bytes, stored and read back transposed as in the 128-row
//    kernel; a step's B fragment is rows 16h + 8s .. +7 of the block.
//  * Wave w owns the 64 columns [64w, 64w+64) and all 256 rows.
__global__ __launch_bounds__(NTHR, 1) void k_dx_bf16_deep(const DxArgs args) {
  constexpr int BM = 256, MI = 8, NM = 16;
  constexpr int KS = 32;                    // K-block width
  constexpr int X_BYTES = BM * KS * 2;      // dy tile [256][32] bf16
  constexpr int W_BYTES = KS * BN * 2;      // weight tile [32][256] bf16
  constexpr int STAGE = X_BYTES + W_BYTES;  // 32 KB
  static_assert(BM * LNF4_EPI_RANK * 2 <= STAGE && BN * LNF4_EPI_RANK * 2 <= STAGE, "LoRA slabs fit a stage");
  static_assert(5 * STAGE <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint8_t sm0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm2[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm3[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sm4[STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  int tm, tn;
  const int n_tiles = args.n_tiles_m * args.n_tiles_n;
  const int split = (int)blockIdx.x / n_tiles;
  tile_coords((int)blockIdx.x - split * n_tiles, args.n_tiles_m, args.n_tiles_n, kGroupM, tm, tn);
  const int M = args.M, N = args.N;
  const int m0 = tm * BM, n0 = tn * BN;
  // the split's 64-row blocks, counted in 32-row blocks
  const int kb64_end = split * args.kb_per_split + args.kb_per_split < args.total_kb
                           ? split * args.kb_per_split + args.kb_per_split : args.total_kb;
  const int kb_beg = 2 * split * args.kb_per_split;
  const int kb_end = 2 * kb64_end;
  const int nc0 = 64 * wave + l32, nc1 = nc0 + 32;

  floatx16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  if (split == 0) dx_bf16_rank_init<MI>(acc, args, m0, n0, sm0, sm1, sm2, tid, l32, h, nc0, nc1);

  // ---- direct global -> LDS loads of one K-block (32 rows of one projection)
  //  * dy: load q of wave w fills tile rows (w*XQ+q)*16 .. +15; lane L -> row +L/4, slot L%4,
  //    which holds chunk (L%4) ^ ((row >> 2) & 3) of the row
  //  * weights: load q of wave w fills rows 2g, 2g+1 (g = w*WQ+q); lane L -> row 2g + L/32,
  //    stored chunk L%32, which holds global chunk (L%32) ^ 4(row & 3) of the row
  //  Rows past the projection's out_f load zeros (the block's resources end there); a block
  //  wholly past it has empty resources.  Columns past N belong to outputs that are dropped.
  constexpr int XQ = X_BYTES / 1024 / 4;
  constexpr int WQ = W_BYTES / 1024 / 4;
  constexpr int NLD = XQ + WQ;
  uint32_t dyr2[XQ], dyc[XQ];
#pragma unroll
  for (int q = 0; q < XQ; ++q) {
    const int row = (wave * XQ + q) * 16 + (lane >> 2);
    dyr2[q] = 2u * (uint32_t)(m0 + row < M ? m0 + row : M - 1);
    dyc[q] = 16u * (uint32_t)((lane & 3) ^ ((row >> 2) & 3));
  }
  uint32_t woff[WQ];
#pragma unroll
  for (int q = 0; q < WQ; ++q) {
    const int row = 2 * (wave * WQ + q) + (lane >> 5);
    const int cg = (lane & 31) ^ (4 * (row & 3));
    woff[q] = 2u * ((uint32_t)row * (uint32_t)N + (uint32_t)(n0 + 8 * cg));
  }

  // the next block to load: its resources end at the projection's last row (rows past
  // out_f load as zeros); blocks past the split, or wholly past out_f, have empty ones
  DxCursor cur = dx_cursor_init<KS>(args, kb_beg);
  rsrc_t wrs_next;  // weight resource of the block whose dy rows went out last
  uint32_t dyo[XQ];
#pragma unroll
  for (int q = 0; q < XQ; ++q) dyo[q] = dyr2[q] * (uint32_t)cur.Kp + dyc[q];
  // A block's loads go out in two parts: its dy rows right after the barrier that frees its
  // stage (step 1 of the block five before it), its weight rows at step 0 of the next
  // block (a burst of all of them at once held up the wave's MFMA issue).  Branch-free: a
  // branch would split the step that issues them, and the interleaving of its MFMAs with
  // its LDS reads is only kept within one basic block.
#define LNF4_DXD_ISSUE_X(SM_)                                                                    \
  {                                                                                              \
    const int live_ = -(int)((cur.kb < kb_end) & (cur.k0 < cur.Kp));                             \
    const int dyn_ = clamp31(((uint64_t)(uint32_t)M * (uint32_t)cur.Kp - (uint32_t)cur.k0) * 2u) & live_; \
    const int wn_ = clamp31((uint64_t)(uint32_t)(cur.Kp - cur.k0) * (2u * (uint32_t)N)) & live_; \
    const rsrc_t dyrs_ = make_rsrc_n(cur.dy + cur.k0, dyn_);                                      \
    wrs_next = make_rsrc_n((const uint16_t*)cur.w + (size_t)cur.k0 * N, wn_);                     \
    _Pragma("unroll") for (int q = 0; q < XQ; ++q)                                               \
      LNF4_BUF_LDS(dyrs_, (SM_) + (wave_u * XQ + q) * 1024, 16, dyo[q], 0);                       \
  }
#define LNF4_DXD_ISSUE_W(SM_)                                                                    \
  {                                                                                              \
    _Pragma("unroll") for (int q = 0; q < WQ; ++q)                                               \
      LNF4_BUF_LDS(wrs_next, (SM_) + X_BYTES + (wave_u * WQ + q) * 1024, 16, woff[q], 0);       \
  }
  // the cursor moves after the step's MFMAs, outside its interleaved region
#define LNF4_DXD_ADVANCE()                                                                       \
  {                                                                                              \
    if (dx_cursor_next<KS>(cur, args)) {                                                         \
      _Pragma("unroll") for (int q = 0; q < XQ; ++q) dyo[q] = dyr2[q] * (uint32_t)cur.Kp + dyc[q]; \
    }                                                                                            \
  }

  typedef short v4s_t __attribute__((ext_vector_type(4)));
  const int tr_c = (lane & 15) >> 2, tr_col = 16 * ((lane & 31) >> 4) + 4 * (lane & 3);
  const int tbo0 = (16 * h + tr_c) * 512 + (((8 * wave + 0 + (tr_col >> 3)) ^ (4 * tr_c)) << 4) + ((tr_col & 7) << 1);
  const int tbo1 = (16 * h + tr_c) * 512 + (((8 * wave + 4 + (tr_col >> 3)) ^ (4 * tr_c)) << 4) + ((tr_col & 7) << 1);
#define LNF4_DXD_TR(SM_, off_) \
  __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)((SM_) + X_BYTES + (off_)))
#define LNF4_DXD_BFRAG(SM_, s_, o_)                                                              \
  ({                                                                                             \
    const v4s_t lo_ = LNF4_DXD_TR(SM_, (o_) + 4096 * (s_));                                      \
    const v4s_t hi_ = LNF4_DXD_TR(SM_, (o_) + 4096 * (s_) + 2048);                               \
    __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo_, hi_, 0, 1, 2, 3, 4, 5, 6, 7));      \
  })
#define LNF4_DXD_AFRAG(SM_, i_, c_)                                                              \
  (*(const bf16x8*)((const uint16_t*)(SM_) + (32 * (i_) + l32) * KS +                           \
                    ((((c_) ^ (((32 * (i_) + l32) >> 2) & 3))) << 3)))

  // prologue: blocks 0 .. 3 and the dy rows of block 4 in flight (its weight rows go out at
  // step 0 of block 0); block 0 visible
  LNF4_DXD_ISSUE_X(sm0);
  LNF4_DXD_ISSUE_W(sm0);
  LNF4_DXD_ADVANCE();
  LNF4_DXD_ISSUE_X(sm1);
  LNF4_DXD_ISSUE_W(sm1);
  LNF4_DXD_ADVANCE();
  LNF4_DXD_ISSUE_X(sm2);
  LNF4_DXD_ISSUE_W(sm2);
  LNF4_DXD_ADVANCE();
  LNF4_DXD_ISSUE_X(sm3);
  LNF4_DXD_ISSUE_W(sm3);
  LNF4_DXD_ADVANCE();
  LNF4_DXD_ISSUE_X(sm4);
  LNF4_DXD_ADVANCE();
  LNF4_WAIT_VM(3 * NLD + XQ);
  __syncthreads();

  bf16x8 ac[MI], an_[MI];
  bf16x8 bc0, bc1, bn0, bn1;
  bc0 = LNF4_DXD_BFRAG(sm0, 0, tbo0);
  bc1 = LNF4_DXD_BFRAG(sm0, 0, tbo1);
#pragma unroll
  for (int i = 0; i < MI; ++i) ac[i] = LNF4_DXD_AFRAG(sm0, i, 2 * h);

  // One 32-row block KB on stage SC; SN holds block KB+1, SP (the stage of KB-1) receives
  // the weight rows of block KB+4 at step 0.  Step 1: every wave's loads of block KB+1 have
  // landed (those of KB+2 .. KB+4 may still be in flight: 3 NLD loads issued after them),
  // the barrier makes KB+1 visible and SC free, and the dy rows of block KB+5 go into SC.
#define LNF4_DXD_BLOCK(KB, SC, SN, SP)                                                             \
  {                                                                                            \
    _Pragma("unroll") for (int s = 0; s < 2; ++s) {                                            \
      __builtin_amdgcn_sched_barrier(0);                                                       \
      if (s == 1) {                                                                            \
        LNF4_WAIT_VM_LGKM0(3 * NLD);                                                           \
        __builtin_amdgcn_s_barrier();                                                          \
        __builtin_amdgcn_sched_barrier(0);                                                     \
        bn0 = LNF4_DXD_BFRAG(SN, 0, tbo0);                                                     \
        bn1 = LNF4_DXD_BFRAG(SN, 0, tbo1);                                                     \
        _Pragma("unroll") for (int i = 0; i < MI; ++i) an_[i] = LNF4_DXD_AFRAG(SN, i, 2 * h);  \
        LNF4_DXD_ISSUE_X(SC);                                                          \
      } else {                                                                                 \
        bn0 = LNF4_DXD_BFRAG(SC, 1, tbo0);                                                     \
        bn1 = LNF4_DXD_BFRAG(SC, 1, tbo1);                                                     \
        _Pragma("unroll") for (int i = 0; i < MI; ++i) an_[i] = LNF4_DXD_AFRAG(SC, i, 2 * h + 1); \
        LNF4_DXD_ISSUE_W(SP);                                                                  \
      }                                                                                        \
      _Pragma("unroll") for (int i = 0; i < MI; ++i) {                                         \
        acc[i][0] = mfma32(ac[i], bc0, acc[i][0]);                                             \
        acc[i][1] = mfma32(ac[i], bc1, acc[i][1]);                                             \
      }                                                                                        \
      _Pragma("unroll") for (int g = 0; g < NM; ++g) {                                         \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                     \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                     \
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                                     \
      }                                                                                        \
      _Pragma("unroll") for (int i = 0; i < MI; ++i) ac[i] = an_[i];                           \
      bc0 = bn0;                                                                               \
      bc1 = bn1;                                                                               \
      if (s == 1) {                                                                            \
        __builtin_amdgcn_sched_barrier(0);                                                     \
        LNF4_DXD_ADVANCE();                                                                    \
      }                                                                                        \
    }                                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                         \
  }

  // whole turns of the ring, one exit test per turn (blocks past the last add zeros)
  for (int kb = kb_beg; kb < kb_end; kb += 5) {
    LNF4_DXD_BLOCK(kb + 0, sm0, sm1, sm4);
    LNF4_DXD_BLOCK(kb + 1, sm1, sm2, sm0);
    LNF4_DXD_BLOCK(kb + 2, sm2, sm3, sm1);
    LNF4_DXD_BLOCK(kb + 3, sm3, sm4, sm2);
    LNF4_DXD_BLOCK(kb + 4, sm4, sm0, sm3);
  }
#undef LNF4_DXD_BLOCK
#undef LNF4_DXD_ISSUE_X
#undef LNF4_DXD_ISSUE_W
#undef LNF4_DXD_ADVANCE
#undef LNF4_DXD_TR
#undef LNF4_DXD_BFRAG
#undef LNF4_DXD_AFRAG

  dx_bf16_store<MI>(acc, args, split, m0, n0, nc0, nc1, h);
}

// Split-K input gradient: dx = bf16(sum of the splits' fp32 sums in split order, plus the
// existing dx when accumulating), 4 elements per thread.
__global__ __launch_bounds__(256) void k_dx_split_sum(const float* __restrict__ part, int n_split, int64_t n,
                                                      int accumulate, uint16_t* __restrict__ dx) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= n) return;
  if (i4 + 4 <= n && ((uintptr_t)dx & 7) == 0) {  // dx itself is only 2-byte aligned in general
    floatx4 s = *(const floatx4*)(part + i4);
    for (int sp = 1; sp < n_split; ++sp) {
      const floatx4 t = *(const floatx4*)(part + (size_t)sp * n + i4);
      s[0] += t[0]; s[1] += t[1]; s[2] += t[2]; s[3] += t[3];
    }
    if (accumulate) {
      const uint2 o = *(const uint2*)(dx + i4);
      s[0] += bf16_lo(o.x); s[1] += bf16_hi(o.x); s[2] += bf16_lo(o.y); s[3] += bf16_hi(o.y);
    }
    *(uint2*)(dx + i4) = make_uint2(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]));
    return;
  }
  for (int64_t i = i4; i < i4 + 4 && i < n; ++i) {
    float s = part[i];
    for (int sp = 1; sp < n_split; ++sp) s += part[(size_t)sp * n + i];
    if (accumulate) s += bf16_to_f32(dx[i]);
    dx[i] = __builtin_bit_cast(uint16_t, (__bf16)s);
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

static int n_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    hipDeviceProp_t prop;
    cus = (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess &&
           prop.multiProcessorCount > 0) ? prop.multiProcessorCount : 256;
  }
  return cus;
}

// K-split plan of an NF4 forward: split count (1: none) and tile height.  128-row tiles when
// they would fill under half of the compute units and K holds at least 32 blocks of 64 (up
// to 4 splits of at least 8 blocks); else 256-row tiles when those fill under half of the
// units and K holds at least 128 blocks (up to 4 splits of at least 64 blocks: a long K
// whose 256-row tiles run more efficiently than twice as many 128-row ones, the Llama-8B
// down projection); in each case as many splits as bring the launch to about one round
static int fwd_split_plan(int M, const int32_t* out_f, int n_proj, int K, int fmt, int& bm) {
  bm = 128;
  if (fmt != 0 || M <= 0 || n_proj < 1) return 1;
  int tn = 0;
  for (int p = 0; p < n_proj; ++p) {
    if (out_f[p] % 4 != 0) return 1;  // the fp32 sums are stored 16 bytes at a time
    tn += (out_f[p] + 255) / 256;
  }
  const int nk = K / 64, cus = n_cus();
  const auto fit = [&](int tiles, int min_blocks) {
    int ks = cus / tiles;
    if (ks > 4) ks = 4;
    if (ks > nk / min_blocks) ks = nk / min_blocks;
    return ks < 2 ? 1 : ks;
  };
  if (pick_bm(M, tn) == 128) {
    const int t128 = ((M + 127) / 128) * tn;
    if (2 * t128 <= cus && nk >= 32) return fit(t128, 8);
  }
  const int t256 = ((M + 255) / 256) * tn;
  if (M > 128 && 2 * t256 <= cus && nk >= 128) {
    const int ks = fit(t256, 64);
    if (ks > 1) bm = 256;
    return ks;
  }
  return 1;
}

int fwd_split_count(int M, const int32_t* out_f, int n_proj, int K, int fmt) {
  int bm;
  return fwd_split_plan(M, out_f, n_proj, K, fmt, bm);
}

size_t fwd_split_bytes(int M, const int32_t* out_f, int n_proj, int K, int fmt) {
  const int ks = fwd_split_count(M, out_f, n_proj, K, fmt);
  if (ks < 2) return 0;
  size_t b = 0;
  for (int p = 0; p < n_proj; ++p) b += (size_t)ks * (size_t)M * (size_t)out_f[p] * 4;
  return b;
}

hipError_t launch_fwd(const FwdArgs& a0, int fmt, hipStream_t s) {
  FwdArgs a = a0;
  if (a.M <= 0 || a.n_tiles_n <= 0) return hipSuccess;
  a.tn_base = 0;
  a.split_block = 0x7fffffff;
  a.tail_m = a.tail_n = a.xcd_f = a.xcd_h = 0;
  const int cus = n_cus();
  if (fmt != 0) {
    // bf16 weights: 256-row tiles with 32-wide K-blocks (a 5-stage ring) where they make
    // at least two rounds over the compute units (the lm_head: 4008 tiles at T = 2048),
    // else 128-row tiles in a 3-stage ring of 64-wide blocks, which keep more units busy
    const int t256 = ((a.M + 255) / 256) * a.n_tiles_n;
    if (t256 >= 2 * cus) {
      a.n_tiles_m = (a.M + 255) / 256;
      hipLaunchKernelGGL(k_fwd_bf16_deep, dim3(t256), dim3(NTHR), 0, s, a);
      return hipGetLastError();
    }
    a.n_tiles_m = (a.M + 127) / 128;
    hipLaunchKernelGGL((k_fwd_bf16<128>), dim3(a.n_tiles_m * a.n_tiles_n), dim3(NTHR), 0, s, a);
    return hipGetLastError();
  }
  const int tn_all = a.n_tiles_n;
  const int tm256 = (a.M + 255) / 256;
  const int t256 = tm256 * tn_all;
  a.ksplit = 1;
  if (a.part != nullptr) {
    int32_t of[kMaxGroup];
    for (int p = 0; p < a.n_proj; ++p) of[p] = a.p[p].out_f;
    int bm = 128;
    const int ks = fwd_split_plan(a.M, of, a.n_proj, a.K, fmt, bm);
    if (ks > 1) {
      // few 128-row tiles over a long K: each tile runs as ks K splits, and a second launch
      // per projection adds the splits' fp32 sums in split order
      a.ksplit = ks;
      a.kb_per_split = (a.K / BK + ks - 1) / ks;
      int64_t off = 0;
      for (int p = 0; p < a.n_proj; ++p) {
        a.p[p].part_off = off;
        off += (int64_t)ks * a.M * a.p[p].out_f;
      }
      a.n_tiles_m = (a.M + bm - 1) / bm;
      if (bm == 256) hipLaunchKernelGGL((k_fwd_nf4<256, 4>), dim3(a.n_tiles_m * a.n_tiles_n * ks), dim3(NTHR), 0, s, a);
      else hipLaunchKernelGGL((k_fwd_nf4<128, 4>), dim3(a.n_tiles_m * a.n_tiles_n * ks), dim3(NTHR), 0, s, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      for (int p = 0; p < a.n_proj; ++p) {
        const int64_t n = (int64_t)a.M * a.p[p].out_f;
        hipLaunchKernelGGL(k_dx_split_sum, dim3((unsigned)(((n + 3) / 4 + 255) / 256)), dim3(256), 0, s,
                           (const float*)(a.part + a.p[p].part_off), ks, n, 0, a.p[p].y);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
      return hipSuccess;
    }
  }
  if (pick_bm(a.M, tn_all) == 128) {
    a.n_tiles_m = (a.M + 127) / 128;
    if (a.n_tiles_m * a.n_tiles_n < cus) {
      // under one round of 128-row tiles: 64-row tiles put twice as many compute units to
      // work (0.5B shapes at T = 2048: q|k|v 96 -> 192 tiles, 10 % faster; each output
      // element is the same sum in the same order)
      a.n_tiles_m = (a.M + 63) / 64;
      hipLaunchKernelGGL((k_fwd_nf4<64, 4>), dim3(a.n_tiles_m * a.n_tiles_n), dim3(NTHR), 0, s, a);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((k_fwd_nf4<128, 4>), dim3(a.n_tiles_m * a.n_tiles_n), dim3(NTHR), 0, s, a);
    return hipGetLastError();
  }
  if (t256 <= cus) {
    // one partial round of tiles, one wave per SIMD (the two-wave form, NW = 8, decodes
    // every code twice: 8B q|k|v, 192 tiles, 0.144 -> 0.134 ms with NW = 4, same bits)
    a.n_tiles_m = tm256;
    hipLaunchKernelGGL((k_fwd_nf4<256, 4>), dim3(t256), dim3(NTHR), 0, s, a);
    return hipGetLastError();
  }
  // Several rounds of 256-row tiles whose last round leaves many compute units idle: the
  // column panels of that last round can run as 128-row tiles in the same launch (a
  // 128-row tile's K loop takes about 0.62 of a 256-row one's: 62 vs 100 us at the 8B
  // gate|up shape).  Chosen when the estimated rounds drop, e.g. 896 tiles = 3.5 rounds on
  // 256 units become 768 + 256 half-height tiles (3.62 estimated rounds instead of 4).
  const int rem = t256 % cus;
  const int tail_n = (rem + tm256 - 1) / tm256;
  const int tm128 = (a.M + 127) / 128;
  const int full = t256 - tail_n * tm256;
  const auto rounds = [cus](int tiles) { return (tiles + cus - 1) / cus; };
  a.n_tiles_m = tm256;
  if (t256 > cus && rem > 0 && full > 0 &&
      rounds(full) + 0.62 * rounds(tm128 * tail_n) < rounds(t256) - 0.2) {
    a.n_tiles_n = tn_all - tail_n;
    a.tail_m = tm128;
    a.tail_n = tail_n;
    const int half = tm128 * tail_n;
    if (half == cus && full >= cus && full % 8 == 0 && half % 8 == 0) {
      // one round of half tiles: the units of four XCDs take theirs first, so those XCDs
      // run half a tile out of step with the other four (each XCD stays in step with
      // itself, so its L2 still serves one set of activation and code panels at a time)
      a.xcd_f = full / 8;
      a.xcd_h = half / 8;
    }
    a.split_block = full;
    hipLaunchKernelGGL((k_fwd_nf4<256, 4>), dim3(full + half), dim3(NTHR), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_fwd_nf4<256, 4>), dim3(t256), dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

// Row-tile height of the input-gradient kernels (bf16 weight tiles are 4x the NF4 bytes:
// their 3-stage ring only fits LDS with 128 rows).
// Row tile of the input gradient.  NF4: 256-row tiles decode each weight element half as
// often per MFMA as 128-row tiles; when they are too few to fill the compute units, K splits
// make up the count (dx_split_count).  Kept only where every split still runs at least 64
// K-blocks: shorter splits lose more to the fp32 partials and the per-tile start than the
// decode (NF4) or the deeper load ring (bf16) saves (measured: gate|up of the 8B shape,
// K = 28672, 2 splits: 17 % faster; K = 4096 or 9728 in 2 or 8 splits: slower).
// bf16 weights take 256-row tiles (k_dx_bf16_deep) only where they need at most two
// splits: with four (the 3B gate|up shape, K = 22016) the extra fp32 partials cost more
// than the tile saves (0.270 against 0.234 ms for 128-row tiles in two splits).
static int dx_bm(int M, int N, int total_kb, int fmt) {
  const int tn = (N + BN - 1) / BN;
  if (fmt == 0 && pick_bm(M, tn) == 256) return 256;
  if (M <= 128) return 128;
  const int tiles = ((M + 255) / 256) * tn;
  int ns = (256 + tiles - 1) / tiles;
  ns = ns > 8 ? 8 : ns;
  if (fmt != 0 && ns > 2) return 128;
  return total_kb / ns >= 64 ? 256 : 128;
}

// Splits of the K space for the input gradient: when the tiles cover less than 3/4 of the
// compute units, split K so that about one wave of workgroups runs, keeping at least 4
// K-blocks per split (at most 8 splits; the 0.5B q|k|v group, 18 K-blocks on 64 tiles,
// takes 4 splits: 76 -> 69 us for its whole backward call).
int dx_split_count(int M, int N, int total_kb, int fmt) {
  if (M <= 0 || N <= 0 || total_kb <= 0) return 1;
  const int bm = dx_bm(M, N, total_kb, fmt);
  const int tiles = ((M + bm - 1) / bm) * ((N + BN - 1) / BN);
  if (tiles >= 192) return 1;
  int ns = (256 + tiles - 1) / tiles;
  const int by_k = total_kb / 4;
  ns = ns < by_k ? ns : by_k;
  ns = ns > 8 ? 8 : ns;
  return ns < 1 ? 1 : ns;
}

size_t dx_split_bytes(int M, int N, int total_kb, int fmt) {
  const int ns = dx_split_count(M, N, total_kb, fmt);
  return ns > 1 ? (size_t)ns * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_dx(const DxArgs& a0, int fmt, hipStream_t s) {
  DxArgs a = a0;
  if (a.M <= 0 || a.N <= 0 || a.total_kb <= 0) return hipSuccess;
  a.n_tiles_n = (a.N + BN - 1) / BN;
  const int bm = dx_bm(a.M, a.N, a.total_kb, fmt);
  a.n_tiles_m = (a.M + bm - 1) / bm;
  const int ns = a.part != nullptr ? dx_split_count(a.M, a.N, a.total_kb, fmt) : 1;
  a.kb_per_split = (a.total_kb + ns - 1) / ns;
  if (ns == 1) a.part = nullptr;
  const dim3 grid(a.n_tiles_m * a.n_tiles_n * ns), block(NTHR);
  if (fmt == 0) {
    if (bm == 256) hipLaunchKernelGGL((k_dxq<256>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_dxq<128>), grid, block, 0, s, a);
  } else {
    if (bm == 256) hipLaunchKernelGGL(k_dx_bf16_deep, grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_dx_bf16<128>), grid, block, 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ns == 1) return e;
  const int64_t n = (int64_t)a.M * a.N;
  const int64_t blocks = (n / 4 + 255) / 256 + 1;
  hipLaunchKernelGGL(k_dx_split_sum, dim3((unsigned)blocks), dim3(256), 0, s, (const float*)a.part, ns, n,
                     a.accumulate, a.dx);
  return hipGetLastError();
}

}  // namespace lnf4
