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
// Layout: one 64-lane wave per (b, c, h) row, four rows (consecutive heads,
// same tokens, so their dt loads share cache lines) per work-group. Each lane
// owns Q/64 consecutive tokens: a serial sum over them, a wave-wide inclusive
// scan of the lane totals (DPP-backed shuffles), a second serial pass, and
// one 16-byte store per lane and output for Q = 256.
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;

template <typename In>
__global__ __launch_bounds__(kThreads) void chunk_cumsum_kernel(const In* __restrict__ dt,
                                                                const float* __restrict__ A,
                                                                float* __restrict__ Acs,
                                                                float* __restrict__ dtq, int T, int H,
                                                                int Q, int nc, long nrows) {
  const long row = long(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= nrows) return;                     // wave-uniform; no barriers in this kernel
  const int lane = threadIdx.x & 63;
  const int h = int(row % H);
  const long bc = row / H;
  const int c = int(bc % nc);
  const int b = int(bc / nc);
  const int per = Q >= 64 ? Q / 64 : 1;         // tokens per lane (1..4)
  const int l0 = lane * per;
  const long t0 = long(c) * Q;
  const float Ah = A[h];
  float d[4] = {0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const long t = t0 + l0 + i;
    if (i < per && l0 + i < Q && t < T) d[i] = to_f32(dt[(size_t(b) * T + t) * H + h]);
    tot += d[i] * Ah;
  }
  float inc = tot;                              // inclusive scan of the lane totals
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  float run = inc - tot;
  float a[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    run += d[i] * Ah;
    a[i] = run;
  }
  const size_t base = ((size_t(b) * H + h) * nc + c) * Q;
  if (per == 4) {
    *reinterpret_cast<f32x4*>(Acs + base + l0) = f32x4{a[0], a[1], a[2], a[3]};
    *reinterpret_cast<f32x4*>(dtq + base + l0) = f32x4{d[0], d[1], d[2], d[3]};
  } else {
    for (int i = 0; i < per; ++i) {
      if (l0 + i < Q) {
        Acs[base + l0 + i] = a[i];
        dtq[base + l0 + i] = d[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_chunk_cumsum(const FwdShape& s, ssd_dtype type, const void* dt, const float* A,
                               float* Acs, float* dtq, hipStream_t st, const StageEv& ev) {
  const long nrows = long(s.b) * s.nc * s.H;
  const long blocks = (nrows + kThreads / 64 - 1) / (kThreads / 64);
  if (type == SSD_BF16)
    hipExtLaunchKernelGGL(chunk_cumsum_kernel<uint16_t>, dim3(unsigned(blocks)), dim3(kThreads), 0, st, ev.start, ev.stop, 0,
                       static_cast<const uint16_t*>(dt), A, Acs, dtq, s.T, s.H, s.Q, s.nc, nrows);
  else
    hipExtLaunchKernelGGL(chunk_cumsum_kernel<float>, dim3(unsigned(blocks)), dim3(kThreads), 0, st, ev.start, ev.stop, 0,
                       static_cast<const float*>(dt), A, Acs, dtq, s.T, s.H, s.Q, s.nc, nrows);
  return hipGetLastError();
}

}  // namespace ssd
