// chunk_state.hip -- the state each chunk produces on its own (zero state in).
//
//   S_c[n, p] = sum_{l in chunk c} B_l[n] * exp(Acs_{Q-1} - Acs_l) * dt_l * x_l[p]
//
// stored transposed, S_c^T [p][n] (n fastest), in [b, nc, H, P, N].
//
// i.e. B^T (N x Q) times diag(decay-to-chunk-end * dt) X (Q x P): the
// final-state row of the semiseparable matrix restricted to one chunk
// (h_T = sum_j abar_{T:j} bbar_j x_j^T with bbar_j = dt_j B_j; youngju.dev
// "Mamba / selective SSM", sections "LTIからSelectionへの切り替え" and
// "State Space Dualityの発見"). These chunk states are what the inter-chunk
// recurrence of the chunked algorithm passes on ("SSDアルゴリズムとチャンク分割").
//
// This translation unit holds the generic fp32-FMA kernel (any dstate and
// headdim up to 256, fp32 or bf16 inputs). The bf16 MFMA kernel for the
// large shapes lives in chunk_state_mfma.hip and is chosen by the launcher.
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kTok = 16;    // tokens staged per step
constexpr int kRows = 32;   // state rows (n) per work-group

template <typename In>
__global__ __launch_bounds__(kThreads) void chunk_state_generic(
    const In* __restrict__ x, const In* __restrict__ B, const float* __restrict__ Acs,
    const float* __restrict__ dtq, float* __restrict__ S, int T, int H, int P, int N, int G, int Q,
    int nc) {
  __shared__ float sB[kTok][kRows];
  __shared__ float sX[kTok][SSD_MAX_HEADDIM];
  const int ntn = (N + kRows - 1) / kRows;
  const int h = blockIdx.x / ntn, n0 = (blockIdx.x % ntn) * kRows;
  const int c = blockIdx.y, b = blockIdx.z;
  const int g = h / (H / G);
  const int tid = threadIdx.x;
  const size_t arow = ((size_t(b) * H + h) * nc + c) * Q;
  const float alast = Acs[arow + Q - 1];
  const long t0 = long(c) * Q;
  const int valid = int(min(long(Q), long(T) - t0));
  const int nout = kRows * P;

  float acc[kRows * SSD_MAX_HEADDIM / kThreads];
#pragma unroll
  for (int k = 0; k < kRows * SSD_MAX_HEADDIM / kThreads; ++k) acc[k] = 0.f;

  for (int s0 = 0; s0 < valid; s0 += kTok) {
    __syncthreads();
    for (int e = tid; e < kTok * kRows; e += kThreads) {
      const int i = e / kRows, j = e % kRows;
      const int s = s0 + i, n = n0 + j;
      sB[i][j] = (s < valid && n < N) ? to_f32(B[((size_t(b) * T + t0 + s) * G + g) * N + n]) : 0.f;
    }
    for (int e = tid; e < kTok * P; e += kThreads) {
      const int i = e / P, p = e % P;
      const int s = s0 + i;
      float v = 0.f;
      if (s < valid) {
        const float w = expf(alast - Acs[arow + s]) * dtq[arow + s];
        v = w * to_f32(x[((size_t(b) * T + t0 + s) * H + h) * P + p]);
      }
      sX[i][p] = v;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kRows * SSD_MAX_HEADDIM / kThreads; ++k) {
      const int e = tid + k * kThreads;
      if (e < nout) {
        const int n = e % kRows, p = e / kRows;
        float a = acc[k];
#pragma unroll
        for (int i = 0; i < kTok; ++i) a += sB[i][n] * sX[i][p];
        acc[k] = a;
      }
    }
  }
  float* out = S + ((size_t(b) * nc + c) * H + h) * size_t(N) * P;
#pragma unroll
  for (int k = 0; k < kRows * SSD_MAX_HEADDIM / kThreads; ++k) {
    const int e = tid + k * kThreads;
    if (e < nout) {
      const int n = n0 + e % kRows, p = e / kRows;
      if (n < N) out[size_t(p) * N + n] = acc[k];
    }
  }
}

}  // namespace

hipError_t launch_chunk_state(const FwdShape& s, ssd_dtype type, const void* x, const void* B,
                              const float* Acs, const float* dtq, float* S, hipStream_t st, const StageEv& ev) {
  const int ntn = (s.N + kRows - 1) / kRows;
  dim3 grid(s.H * ntn, s.nc, s.b);
  if (type == SSD_BF16)
    hipExtLaunchKernelGGL(chunk_state_generic<uint16_t>, grid, dim3(kThreads), 0, st, ev.start, ev.stop, 0,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(B), Acs, dtq, S,
                       s.T, s.H, s.P, s.N, s.G, s.Q, s.nc);
  else
    hipExtLaunchKernelGGL(chunk_state_generic<float>, grid, dim3(kThreads), 0, st, ev.start, ev.stop, 0,
                       static_cast<const float*>(x), static_cast<const float*>(B), Acs, dtq, S, s.T,
                       s.H, s.P, s.N, s.G, s.Q, s.nc);
  return hipGetLastError();
}

}  // namespace ssd
