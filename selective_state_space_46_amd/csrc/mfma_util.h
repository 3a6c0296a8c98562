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

// Lane moves within a wave by DPP (no LDS traffic, unlike a shuffle, which
// goes through the LDS crossbar and queues behind its other work). CTRL is the
// DPP control (0x111 + n - 1: row_shr:n; 0x142: row_bcast:15; 0x143:
// row_bcast:31) and ROWS the rows of 16 lanes written; every other lane,
// and a lane whose source lies outside its row, receives 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8
// lanes give the sums inside each row of 16; broadcasting lane 15's value to
// row 1 and lane 47's to row 3, then lane 31's to rows 2 and 3, carries the
// totals of the rows before.
__device__ __forceinline__ float wave_incl_scan(float x) {
  x += dpp_move<0x111, 0xF>(x);
  x += dpp_move<0x112, 0xF>(x);
  x += dpp_move<0x114, 0xF>(x);
  x += dpp_move<0x118, 0xF>(x);
  x += dpp_move<0x142, 0xA>(x);
  x += dpp_move<0x143, 0xC>(x);
  return x;
}

// ---------------------------------------------------------------------------
// LDS tiles in natural (row-major, token-major) order, read transposed.
//
// ds_read_b64_tr_b16 (gfx950) works on groups of 16 lanes: destination lane
// 4a + e of a group receives element e (16-bit) of the 8-byte chunks that
// lanes a, a+4, a+8, a+12 of the group address (checked on MI355X). If lane
// q of a group addresses row kb + q/4, columns m0 + 4 (q%4) .. +4, lane q
// receives rows kb .. kb+3 of column m0 + q: four consecutive k of one MFMA
// row/column. Two such reads give one 8-element operand fragment.
//
// Rows are stored as 16-byte chunks, chunk c of row r at chunk c ^ swz(r).
// LDS has 64 banks of 4 bytes and serves an 8-byte read 32 lanes per cycle
// (measured on MI355X with SQ_LDS_BANK_CONFLICT). Transposed reads: 32 lanes
// read four rows kb .. kb+3 (kb % 4 == 0), 64 bytes (four aligned chunks) of
// each, which must cover all 64 banks. With RB chunks per row:
//   RB = 4  (64 B rows):  rows start 16 banks apart            -> swz = 0
//   RB = 8  (128 B rows): rows r, r+1 differ by 32 banks        -> swz = 4 ((r >> 1) & 1)
//   RB >= 16 (256 B, 512 B rows): every row starts at bank 0    -> swz = 4 (r & 3)
// ROWS = true adds a second access shape, row reads: 32 lanes read 8 bytes of
// the same chunk in 32 consecutive rows (the chunk_scan epilogue). Under the
// swizzle above they are 8-way conflicts; XOR-ing (r >> 2) & 3 into the low
// chunk bits as well rotates chunks inside an aligned group of four across
// row quads, which brings them to 2-way (the floor: 32 lanes x 8 bytes of one
// half-chunk column fill only 32 two-bank slots) and leaves transposed reads
// conflict-free. It costs a few more address instructions where the row
// varies, so tiles without row reads keep the plain form.
// Row-major 16-byte writes of whole rows are conflict-free under both (any
// chunk permutation inside a row keeps them so).
template <int RB, bool ROWS = false>
__device__ __forceinline__ int lds_swz(int r) {
  const int rot = ROWS ? ((r >> 2) & 3) : 0;
  if constexpr (RB <= 4) return rot;
  else if constexpr (RB == 8) return (4 * ((r >> 1) & 1)) | rot;
  else return (4 * (r & 3)) | rot;
}

// Element offset of (row r, column col) in a swizzled tile with RB chunks/row.
template <int RB, bool ROWS = false>
__device__ __forceinline__ int lds_off(int r, int col) {
  return r * (RB * 8) + (((col >> 3) ^ lds_swz<RB, ROWS>(r)) << 3) + (col & 7);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* tile, int elem_off) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  // the tile lives in LDS; cast the generic pointer to the local address space
  const __attribute__((address_space(3))) char* p =
      (const __attribute__((address_space(3))) char*)(tile) + 2 * elem_off;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// One 32x32x16 operand fragment (8 consecutive k for MFMA row/column L % 32 of
// the 32-wide block starting at column m0) from a swizzled natural tile whose
// rows are the k axis: k rows kb1 .. kb1+3 and kb2 .. kb2+3 (kb1, kb2 already
// include this lane's 8 (L/32) offset, so any k permutation shared with the
// other operand can be expressed).
template <int RB, bool ROWS = false>
__device__ __forceinline__ u32x4 frag_tr(const uint16_t* tile, int kb1, int kb2, int m0, int lane) {
  const int q = lane & 15, m = m0 + 16 * ((lane >> 4) & 1) + 4 * (q & 3);
  const u32x2 lo = lds_read_tr16(tile, lds_off<RB, ROWS>(kb1 + (q >> 2), m));
  const u32x2 hi = lds_read_tr16(tile, lds_off<RB, ROWS>(kb2 + (q >> 2), m));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Keep `v` when `keep`, else zeros. Loads stay unconditional (their row index
// is clamped into the tensor by the caller) so the compiler can issue a batch
// of them back to back; a branch around each load would serialise them.
__device__ __forceinline__ u32x4 keep_or_zero(bool keep, const u32x4& v) {
  return keep ? v : u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// Direct global -> LDS copies and the waits around them.
// ---------------------------------------------------------------------------

// vmcnt(n), the other counters left alone (low four bits of n in bits 3..0,
// high two in bits 15..14)
// v, hidden from the optimizer: values derived from it inside a loop are
// recomputed there instead of being hoisted out of the loop and held in
// registers for its whole length (lane-dependent addresses of unrolled
// accesses would otherwise take more registers than the MFMA accumulators).
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Work-group barrier for LDS traffic only (the waves of this launch share
// nothing else through memory): this wave's LDS operations complete, then
// the barrier; the memory clobber keeps the compiler from moving memory
// accesses across it. Unlike __syncthreads it does not make each wave wait
// for its slice copies still in flight, which the copy protocol waits for
// by count instead.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One wave's direct copy of 64 x 16 bytes from global memory into LDS: lane
// L's 16 bytes land at dst + 16 L (dst wave-uniform; checked on MI355X).
__device__ __forceinline__ void copy_to_lds16(const uint16_t* src, uint16_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(dst), 16, 0, 0);
}

}  // namespace ssd
