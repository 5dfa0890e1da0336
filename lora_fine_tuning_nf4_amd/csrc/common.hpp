// Device-side building blocks shared by the lnf4 kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf4_table.hpp"

namespace lnf4 {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// native 4 x 32-bit vector: register arrays of these are split into registers by SROA
// (arrays of the HIP uint4 wrapper struct can stay in private memory)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource over [p, p + bytes) for the direct-to-LDS buffer loads: a 32-bit
// per-lane offset plus a wave-uniform offset address the data with no per-lane 64-bit
// arithmetic, and a load whose per-lane offset reaches past `bytes` returns zeros.
// (dword 3 = 0x00020000: the untyped 32-bit format of gfx9-class buffer descriptors)
// The host pass of hipcc only parses kernel bodies; it has no buffer-resource type, and a
// kernel it cannot parse gets no launch stub, so it sees an inert stand-in.
typedef __attribute__((address_space(3))) void* lds_ptr;
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (bytes < 0 ? 0 : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}
// the same with a byte count already in [0, 2^31)
__device__ __forceinline__ rsrc_t make_rsrc_n(const void* p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}
#define LNF4_BUF_LDS(rsrc_, lds_, size_, voff_, soff_) \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_, (lds_ptr)(lds_), size_, voff_, soff_, 0, 0)
#else
typedef const void* rsrc_t;
__device__ inline rsrc_t make_rsrc(const void* p, int64_t) { return p; }
__device__ inline rsrc_t make_rsrc_n(const void* p, int) { return p; }
#define LNF4_BUF_LDS(rsrc_, lds_, size_, voff_, soff_) ((void)(rsrc_), (void)(lds_), (void)(voff_), (void)(soff_))
#endif

// Buffer loads into registers.  The host pass gets inert stand-ins, as for the
// direct-to-LDS loads.
#if defined(__HIP_DEVICE_COMPILE__)
#define LNF4_BUF_LD128(rsrc_, voff_, soff_) __builtin_amdgcn_raw_buffer_load_b128(rsrc_, voff_, soff_, 0)
#define LNF4_BUF_LD32(rsrc_, voff_, soff_) __builtin_amdgcn_raw_buffer_load_b32(rsrc_, voff_, soff_, 0)
#else
#define LNF4_BUF_LD128(rsrc_, voff_, soff_) ((void)(rsrc_), (void)(voff_), (void)(soff_), u32x4{0u, 0u, 0u, 0u})
#define LNF4_BUF_LD32(rsrc_, voff_, soff_) ((void)(rsrc_), (void)(voff_), (void)(soff_), 0u)
#endif

// Two fp32 -> packed bf16 pair, round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
// `lo` lands in bits 0..15 (the lower address), `hi` in bits 16..31.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Decode one dword of NF4 codes (8 elements, element 2b in the high nibble of byte b)
// with one block scale: out dword q = bf16(T[c_2q]*a) | bf16(T[c_2q+1]*a) << 16.
// `lut` is the code table in LDS (16 fp32; every lane reads one of 16 words, so the
// reads broadcast without bank conflicts).  One fp32 product per element, then RNE.
__device__ __forceinline__ void decode8(uint32_t w, float a, const float* lut, uint32_t out[4]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t hi = (w >> (8 * b + 4)) & 15u;
    const uint32_t lo = (w >> (8 * b)) & 15u;
    const float f0 = lut[hi] * a;
    const float f1 = lut[lo] * a;
    out[b] = pack_bf16x2(f0, f1);
  }
}

// Same decode, returning fp32 products for element e = 0..7 of the dword.
__device__ __forceinline__ void decode8_f32(uint32_t w, float a, const float* lut, float out[8]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    out[2 * b] = lut[(w >> (8 * b + 4)) & 15u] * a;
    out[2 * b + 1] = lut[(w >> (8 * b)) & 15u] * a;
  }
}

// Logical block index -> tile index so that the blocks the hardware places on one XCD
// (block b runs on XCD b % 8) get one contiguous range of tiles: tiles that share an
// operand then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int per = nb >> 3, rem = nb & 7;
  const int x = b & 7, i = b >> 3;
  return x * per + (x < rem ? x : rem) + i;
}

// Tile coordinates of a logical block.  The blocks of one XCD take a contiguous range of
// the tile sequence (xcd_remap), and the sequence walks groups of gm row-tiles across all
// column-tiles, so the 32 blocks resident on one XCD at a time cover gm row-panels and
// 32/gm column-panels: each activation panel and each weight panel they stream is read
// from HBM once for the XCD and shared through its L2.
__device__ __forceinline__ void tile_from_seq(int t, int n_m, int n_n, int gm, int& tm, int& tn) {
  const int per_group = gm * n_n;
  const int g = t / per_group, first = g * gm;
  const int gsz = n_m - first < gm ? n_m - first : gm;
  const int r = t - g * per_group;
  tm = first + r % gsz;
  tn = r / gsz;
}
__device__ __forceinline__ void tile_coords(int b, int n_m, int n_n, int gm, int& tm, int& tn) {
  tile_from_seq(xcd_remap(b, n_m * n_n), n_m, n_n, gm, tm, tn);
}

}  // namespace lnf4
