// chunk_scores.hip -- C B^T inside each chunk, once per B/C group.
//
//   CB[l][s] = C_l . B_s      for l, s in the same chunk, s <= l (32 x 32 tiles)
//
// These are the dot products of the semiseparable matrix M_ij = C_i^T
// abar_{i:j} B_j before its decay (youngju.dev "Mamba / selective SSM",
// section "State Space Dualityの発見"); they depend only on B and C, which the
// heads of one group share (Qiita "Mamba-2" article, section 4.1: heads like
// multi-head attention, B/C per group). chunk_scan applies the per-head decay
// and causal mask to them.
//
// One wave per (batch, chunk, group, 32-row block l). C_l stays in registers
// (k = dstate, loaded straight from HBM: B and C rows are dstate-contiguous),
// the B rows of each column block s <= l stream through a double buffer, and
// each tile is written as bf16 in MFMA result order: tile (s, l) is 64 lanes x
// 16 values, lane L holding rows 8(r/4) + 4(L/32) + r%4 of column L%32, i.e.
// exactly the B-operand fragments chunk_scan feeds to its next MFMA, loaded
// there with two coalesced 16-byte reads per lane.
//
// Layout: CB [b, nc, G, ntile, 64, 16] bf16 with ntile = lpc(lpc+1)/2,
// lpc = Q/32, tile (s, l) of a chunk at index l(l+1)/2 + s.
#include "mfma_util.h"

namespace ssd {
namespace {

constexpr int kThreads = 64;

template <int N>
__global__ __launch_bounds__(kThreads) void chunk_scores_kernel(const uint16_t* __restrict__ Bm,
                                                                const uint16_t* __restrict__ Cm,
                                                                uint16_t* __restrict__ CB, int T,
                                                                int G, int Q, int nc) {
  const int lpc = Q / 32;
  const int ntile = lpc * (lpc + 1) / 2;
  int bid = blockIdx.x;
  const int i = bid % lpc; bid /= lpc;        // row block inside the chunk
  const int g = bid % G; bid /= G;
  const int c = bid % nc;
  const int b = bid / nc;
  const int lane = threadIdx.x, l32 = lane & 31, g2 = lane >> 5;
  const int tc0 = c * Q;                       // first token of the chunk
  if (tc0 + 32 * i >= T) return;               // block entirely past the end: never read

  const int tl = tc0 + 32 * i + l32;
  u32x4 cf[N / 16];
  {
    const uint16_t* cr = Cm + ((size_t(b) * T + min(tl, T - 1)) * G + g) * N + 8 * g2;
#pragma unroll
    for (int ks = 0; ks < N / 16; ++ks) cf[ks] = load16(cr + 16 * ks);
#pragma unroll
    for (int ks = 0; ks < N / 16; ++ks) cf[ks] = keep_or_zero(tl < T, cf[ks]);
  }
  auto load_b = [&](int j, u32x4 (&bf)[N / 16]) {
    const int ts = tc0 + 32 * j + l32;
    const uint16_t* br = Bm + ((size_t(b) * T + min(ts, T - 1)) * G + g) * N + 8 * g2;
#pragma unroll
    for (int ks = 0; ks < N / 16; ++ks) bf[ks] = load16(br + 16 * ks);
  };
  constexpr bool kPrefetch = N <= 128;
  u32x4 bnext[N / 16];
  if (kPrefetch) load_b(0, bnext);
  uint16_t* out = CB + (((size_t(b) * nc + c) * G + g) * ntile + size_t(i) * (i + 1) / 2) * 1024 +
                  size_t(lane) * 16;
  for (int j = 0; j <= i; ++j) {
    u32x4 bcur[N / 16];
    if (kPrefetch) {
#pragma unroll
      for (int ks = 0; ks < N / 16; ++ks) bcur[ks] = bnext[ks];
      if (j < i) load_b(j + 1, bnext);
    } else {
      load_b(j, bcur);
    }
    const bool jin = tc0 + 32 * j + l32 < T;
#pragma unroll
    for (int ks = 0; ks < N / 16; ++ks) bcur[ks] = keep_or_zero(jin, bcur[ks]);
    f32x16 acc = zero16();
#pragma unroll
    for (int ks = 0; ks < N / 16; ++ks) acc = mfma32x32x16(bcur[ks], cf[ks], acc);  // rows s, column l
    u32x4 lo, hi;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      lo[m] = pack_bf16x2(acc[2 * m], acc[2 * m + 1]);
      hi[m] = pack_bf16x2(acc[8 + 2 * m], acc[8 + 2 * m + 1]);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(out + size_t(j) * 1024);
    dst[0] = lo;
    dst[1] = hi;
  }
}

template <int N>
hipError_t launch_n(const FwdShape& s, const void* B, const void* C, uint16_t* CB, hipStream_t st) {
  const long blocks = long(s.b) * s.nc * s.G * (s.Q / 32);
  hipLaunchKernelGGL((chunk_scores_kernel<N>), dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                     static_cast<const uint16_t*>(B), static_cast<const uint16_t*>(C), CB, s.T, s.G,
                     s.Q, s.nc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_scores(const FwdShape& s, const void* B, const void* C, uint16_t* CB,
                               hipStream_t st) {
  switch (s.N) {
    case 32: return launch_n<32>(s, B, C, CB, st);
    case 64: return launch_n<64>(s, B, C, CB, st);
    case 128: return launch_n<128>(s, B, C, CB, st);
    case 256: return launch_n<256>(s, B, C, CB, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace ssd
