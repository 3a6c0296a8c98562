// chunk_cumsum.hip -- in-chunk inclusive prefix sum of dt*A_h.
//
// For every (b, h, chunk c) and position l of the chunk:
//   Acs[b,h,c,l] = sum_{k=0..l} dt[b, cQ+k, h] * A[h]
//   dtq[b,h,c,l] = dt[b, cQ+l, h]            (both use dt = 0 past the end)
// The segment sums sum_{k=j+1..i} dt_k A = Acs_i - Acs_j are the exponents of
// the decay products abar_{i:j} in the semiseparable matrix
// M_ij = C_i^T abar_{i:j} B_j (youngju.dev "Mamba / selective SSM", section
// "State Space Dualityの発見"). The per-chunk cumsum of dt is the first step of
// the chunked algorithm on the same page ("SSDアルゴリズムとチャンク分割").
// Tokens past the end of the sequence use dt = 0, which blocks the state
// update (same page, "デバッグチェックリスト").
//
// Layout: one 64-lane wave per (b, h, c) row. dt is [b, T, H] (heads fastest),
// so a work-group stages a [Q x 16 heads] tile of dt through LDS with
// coalesced row reads, then each wave scans one head's column: a serial sum
// over the lane's Q/64 consecutive tokens, a wave-wide inclusive scan of the
// lane totals (DPP-backed shuffles), and a second serial pass.
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kHeadsPerBlock = 16;
constexpr int kThreads = 256;  // 4 waves; each wave scans kHeadsPerBlock/4 heads

template <typename In>
__global__ __launch_bounds__(kThreads) void chunk_cumsum_kernel(const In* __restrict__ dt,
                                                                const float* __restrict__ A,
                                                                float* __restrict__ Acs,
                                                                float* __restrict__ dtq, int T, int H,
                                                                int Q, int nc) {
  __shared__ float tile[256][kHeadsPerBlock + 1];
  const int c = blockIdx.x;
  const int h0 = blockIdx.y * kHeadsPerBlock;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int nh = min(kHeadsPerBlock, H - h0);
  const long t0 = long(c) * Q;

  // Stage dt[b, t0 .. t0+Q, h0 .. h0+nh] (zero past the end of the sequence).
  for (int e = tid; e < Q * kHeadsPerBlock; e += kThreads) {
    const int l = e / kHeadsPerBlock, j = e % kHeadsPerBlock;
    float v = 0.f;
    if (j < nh && t0 + l < T) v = to_f32(dt[(size_t(b) * T + t0 + l) * H + h0 + j]);
    tile[l][j] = v;
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  const int per = Q >= 64 ? Q / 64 : 1;  // tokens per lane (1..4)
  const int l0 = lane * per;
  for (int j = wave; j < nh; j += kThreads / 64) {
    const int h = h0 + j;
    const float Ah = A[h];
    float tot = 0.f;
    for (int i = 0; i < per; ++i)
      if (l0 + i < Q) tot += tile[l0 + i][j] * Ah;
    // inclusive scan of the lane totals across the wave
    float inc = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(inc, off, 64);
      if (lane >= off) inc += o;
    }
    float run = inc - tot;
    const size_t row = ((size_t(b) * H + h) * nc + c) * Q;
    for (int i = 0; i < per; ++i) {
      const int l = l0 + i;
      if (l < Q) {
        const float d = tile[l][j];
        run += d * Ah;
        Acs[row + l] = run;
        dtq[row + l] = d;
      }
    }
  }
}

}  // namespace

hipError_t launch_chunk_cumsum(const FwdShape& s, ssd_dtype type, const void* dt, const float* A,
                               float* Acs, float* dtq, hipStream_t st) {
  dim3 grid(s.nc, (s.H + kHeadsPerBlock - 1) / kHeadsPerBlock, s.b);
  if (type == SSD_BF16)
    hipLaunchKernelGGL(chunk_cumsum_kernel<uint16_t>, grid, dim3(kThreads), 0, st,
                       static_cast<const uint16_t*>(dt), A, Acs, dtq, s.T, s.H, s.Q, s.nc);
  else
    hipLaunchKernelGGL(chunk_cumsum_kernel<float>, grid, dim3(kThreads), 0, st,
                       static_cast<const float*>(dt), A, Acs, dtq, s.T, s.H, s.Q, s.nc);
  return hipGetLastError();
}

}  // namespace ssd
