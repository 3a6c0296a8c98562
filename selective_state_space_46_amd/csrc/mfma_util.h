// mfma_util.h -- CDNA4 (gfx950) matrix-core helpers for the bf16 kernels.
//
// v_mfma_f32_32x32x16_bf16 lane layout (wave64), checked on MI355X:
//   A (32 x 16):  lane L holds A[L % 32][8 * (L / 32) + j],  j = 0..7
//   B (16 x 32):  lane L holds B[8 * (L / 32) + j][L % 32],  j = 0..7
//   C (32 x 32):  lane L, register r holds C[8 * (r / 4) + 4 * (L / 32) + r % 4][L % 32]
// Because the k order inside one instruction is a sum, any permutation of k
// applied to both A and B gives the same product; the kernels use this to feed
// a C tile straight back as an A operand (see chunk_scan_mfma.hip).
#pragma once

#include "ssd_internal.h"

namespace ssd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Two fp32 -> packed bf16 pair (round to nearest even; the gfx950 hardware
// conversion).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = __builtin_convertvector(f32x2{lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 x 8 transpose of 16-bit elements held as 8 rows of 4 dwords: in[i] holds
// row i (elements 2k, 2k+1 in dword k); out[j] receives column j the same way.
__device__ __forceinline__ void transpose8x8_b16(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t a = in[2 * m][j / 2], b = in[2 * m + 1][j / 2];
      out[j][m] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
  }
}

__device__ __forceinline__ u32x4 load16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// Keep `v` when `keep`, else zeros. Loads stay unconditional (their row index
// is clamped into the tensor by the caller) so the compiler can issue a batch
// of them back to back; a branch around each load would serialise them.
__device__ __forceinline__ u32x4 keep_or_zero(bool keep, const u32x4& v) {
  return keep ? v : u32x4{0u, 0u, 0u, 0u};
}

}  // namespace ssd
