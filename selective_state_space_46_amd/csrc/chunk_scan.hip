// chunk_scan.hip -- outputs of one chunk given the state entering it.
//
//   y_l = sum_{s <= l, s in chunk} (C_l . B_s) exp(Acs_l - Acs_s) dt_s x_s     (intra-chunk)
//       + exp(Acs_l) C_l^T H_c                                                 (state entering)
//       + D_h x_l
//
// The intra-chunk part is the chunk's diagonal block of y = M x with the
// semiseparable M_ij = C_i^T abar_{i:j} B_j (youngju.dev "Mamba / selective
// SSM", section "State Space Dualityの発見"): an attention-like product where
// the causal mask and the decay exp(segment sum) replace softmax. The second
// term carries the earlier chunks' contribution through the passed state
// ("SSDアルゴリズムとチャンク分割" on the same page). The mask is applied before
// the exponential, so exp only ever sees Acs_l - Acs_s <= 0.
//
// This translation unit holds the generic fp32-FMA kernel; the bf16 MFMA
// kernel for the large shapes lives in chunk_scan_mfma.hip.
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 16;  // output rows (tokens) per work-group

template <typename In>
__global__ __launch_bounds__(kThreads) void chunk_scan_generic(
    const In* __restrict__ x, const In* __restrict__ B, const In* __restrict__ C,
    const float* __restrict__ Acs, const float* __restrict__ dtq, const float* __restrict__ Hst,
    const float* __restrict__ D, In* __restrict__ y, int T, int H, int P, int N, int G, int Q,
    int nc) {
  __shared__ float sc[kRows][256];                // decayed, masked scores
  __shared__ float sC[kRows][SSD_MAX_DSTATE];     // C rows of this block
  const int nrb = Q / kRows;
  const int h = blockIdx.x / nrb, r0 = (blockIdx.x % nrb) * kRows;
  const int c = blockIdx.y, b = blockIdx.z;
  const int g = h / (H / G);
  const int tid = threadIdx.x;
  const long t0 = long(c) * Q;
  const int valid = int(min(long(Q), long(T) - t0));
  if (r0 >= valid) return;  // the whole work-group leaves together
  const size_t arow = ((size_t(b) * H + h) * nc + c) * Q;

  for (int e = tid; e < kRows * N; e += kThreads) {
    const int i = e / N, n = e % N;
    const int l = r0 + i;
    sC[i][n] = l < valid ? to_f32(C[((size_t(b) * T + t0 + l) * G + g) * N + n]) : 0.f;
  }
  __syncthreads();

  const int smax = min(r0 + kRows, valid);  // columns s = 0 .. smax-1
  for (int e = tid; e < kRows * smax; e += kThreads) {
    const int i = e / smax, s = e % smax;
    const int l = r0 + i;
    float v = 0.f;
    if (s <= l && l < valid) {
      const In* Bs = B + ((size_t(b) * T + t0 + s) * G + g) * N;
      float dot = 0.f;
      for (int n = 0; n < N; ++n) dot += sC[i][n] * to_f32(Bs[n]);
      v = dot * expf(Acs[arow + l] - Acs[arow + s]) * dtq[arow + s];
    }
    sc[i][s] = v;
  }
  __syncthreads();

  const float Dh = D ? D[h] : 0.f;
  const float* Hc = Hst + ((size_t(b) * nc + c) * H + h) * size_t(N) * P;
  for (int e = tid; e < kRows * P; e += kThreads) {
    const int i = e / P, p = e % P;
    const int l = r0 + i;
    if (l >= valid) continue;
    float acc = 0.f;
    for (int s = 0; s <= l; ++s) acc += sc[i][s] * to_f32(x[((size_t(b) * T + t0 + s) * H + h) * P + p]);
    float accH = 0.f;
    for (int n = 0; n < N; ++n) accH += sC[i][n] * Hc[size_t(p) * N + n];
    const size_t xi = ((size_t(b) * T + t0 + l) * H + h) * P + p;
    const float out = acc + expf(Acs[arow + l]) * accH + Dh * to_f32(x[xi]);
    y[xi] = from_f32<In>(out);
  }
}

}  // namespace

hipError_t launch_chunk_scan(const FwdShape& s, ssd_dtype type, bool mfma, const void* x,
                             const void* B, const void* C, const float* Acs, const float* dtq,
                             const float* Hst, const uint16_t* Hb, const uint16_t* CB, const uint16_t* Cf,
                             const float* D, void* y, hipStream_t st, const StageEv& ev) {
  if (mfma) return launch_chunk_scan_mfma(s, x, CB, Cf, Acs, dtq, Hb, D, y, nullptr, st, ev);
  dim3 grid(s.H * (s.Q / kRows), s.nc, s.b);
  if (type == SSD_BF16)
    hipExtLaunchKernelGGL(chunk_scan_generic<uint16_t>, grid, dim3(kThreads), 0, st, ev.start, ev.stop, 0,
                       static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(B),
                       static_cast<const uint16_t*>(C), Acs, dtq, Hst, D,
                       static_cast<uint16_t*>(y), s.T, s.H, s.P, s.N, s.G, s.Q, s.nc);
  else
    hipExtLaunchKernelGGL(chunk_scan_generic<float>, grid, dim3(kThreads), 0, st, ev.start, ev.stop, 0,
                       static_cast<const float*>(x), static_cast<const float*>(B),
                       static_cast<const float*>(C), Acs, dtq, Hst, D, static_cast<float*>(y), s.T,
                       s.H, s.P, s.N, s.G, s.Q, s.nc);
  return hipGetLastError();
}

}  // namespace ssd
