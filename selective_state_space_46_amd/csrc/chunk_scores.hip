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
// One wave per tile (batch, chunk, group, 32-row block l, 32-column block
// s <= l), four tiles per work-group: the C_l and B_s rows load straight from
// HBM/L2 (k = dstate; B and C rows are dstate-contiguous) as one batch, eight
// (dstate 128) MFMAs follow, and the tile is written as bf16 in MFMA result
// order: tile (s, l) is 64 lanes x
// 16 values, lane L holding rows 8(r/4) + 4(L/32) + r%4 of column L%32, i.e.
// exactly the B-operand fragments chunk_scan feeds to its next MFMA, loaded
// there with two coalesced 16-byte reads per lane.
//
// Layout: CB [b, nc, G, ntile, 64, 16] bf16 with ntile = lpc(lpc+1)/2,
// lpc = Q/32, tile (s, l) of a chunk at index l(l+1)/2 + s.
#include "mfma_util.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;  // four tiles per work-group, one per wave

template <int N>
__global__ __launch_bounds__(kThreads) void chunk_scores_kernel(const uint16_t* __restrict__ Bm,
                                                                const uint16_t* __restrict__ Cm,
                                                                uint16_t* __restrict__ CB, int T,
                                                                int G, int Q, int nc, long ntot) {
  const int lpc = Q / 32;
  const int ntile = lpc * (lpc + 1) / 2;
  const int lane = threadIdx.x & 63, l32 = lane & 31, g2 = lane >> 5;
  const long wid = long(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (wid >= ntot) return;                      // wave-uniform; no barriers in this kernel
  long rest = wid;
  const int ti = int(rest % ntile); rest /= ntile;
  const int g = int(rest % G); rest /= G;
  const int c = int(rest % nc);
  const int b = int(rest / nc);
  int i = 0;                                    // tile ti = i (i + 1) / 2 + j, j <= i
  while ((i + 1) * (i + 2) / 2 <= ti) ++i;
  const int j = ti - i * (i + 1) / 2;
  const int tc0 = c * Q;                        // first token of the chunk
  if (tc0 + 32 * i >= T) return;                // row block past the end: never read

  const int tl = tc0 + 32 * i + l32, ts = tc0 + 32 * j + l32;
  const uint16_t* cr = Cm + ((size_t(b) * T + min(tl, T - 1)) * G + g) * N + 8 * g2;
  const uint16_t* br = Bm + ((size_t(b) * T + min(ts, T - 1)) * G + g) * N + 8 * g2;
  u32x4 cf[N / 16], bf[N / 16];
#pragma unroll
  for (int ks = 0; ks < N / 16; ++ks) {
    cf[ks] = load16(cr + 16 * ks);
    bf[ks] = load16(br + 16 * ks);
  }
  f32x16 acc = zero16();
#pragma unroll
  for (int ks = 0; ks < N / 16; ++ks)
    acc = mfma32x32x16(keep_or_zero(ts < T, bf[ks]), keep_or_zero(tl < T, cf[ks]), acc);  // rows s, column l
  u32x4 lo, hi;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    lo[m] = pack_bf16x2(acc[2 * m], acc[2 * m + 1]);
    hi[m] = pack_bf16x2(acc[8 + 2 * m], acc[8 + 2 * m + 1]);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(CB + (((size_t(b) * nc + c) * G + g) * ntile + ti) * 1024 +
                                        size_t(lane) * 16);
  dst[0] = lo;
  dst[1] = hi;
}

template <int N>
hipError_t launch_n(const FwdShape& s, const void* B, const void* C, uint16_t* CB, hipStream_t st) {
  const int lpc = s.Q / 32;
  const long ntot = long(s.b) * s.nc * s.G * (lpc * (lpc + 1) / 2);
  const long blocks = (ntot + kThreads / 64 - 1) / (kThreads / 64);
  hipLaunchKernelGGL((chunk_scores_kernel<N>), dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                     static_cast<const uint16_t*>(B), static_cast<const uint16_t*>(C), CB, s.T, s.G,
                     s.Q, s.nc, ntot);
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
