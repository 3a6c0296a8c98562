// state_update.hip -- the recurrent single-token mode (decode).
//
//   h <- exp(dt A_h) h + (dt B) x^T ;   y = C^T h + D_h x       (in place on h)
//
// One step of h_t = abar_t h_{t-1} + bbar_t x_t, y_t = C_t h_t with
// abar = exp(dt A), bbar = dt B (youngju.dev "Mamba / selective SSM", section
// "LTIからSelectionへの切り替え"): the constant-memory inference form of the
// layer (Qiita "Mamba-2" article, section 3.3; waylandz LLM book ch. 32,
// section 32.2.4).
//
// HBM-bound: every step reads and writes the whole fp32 state once
// (8 bytes per element, ~0.5 flop/byte). One work-group per (b, h) state of
// N x P fp32; each thread owns 4 consecutive columns (one f32x4) of a
// strided set of rows, so a wave reads and writes whole rows contiguously.
// The column sums over n are reduced across the work-group through LDS in a
// fixed order (deterministic).
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;

template <typename In>
__global__ __launch_bounds__(kThreads) void state_update_vec4(
    float* __restrict__ state, const In* __restrict__ x, const In* __restrict__ dt,
    const float* __restrict__ A, const In* __restrict__ B, const In* __restrict__ C,
    const float* __restrict__ D, In* __restrict__ y, int H, int P, int N, int G) {
  __shared__ f32x4 part[kThreads];
  __shared__ float sB[SSD_MAX_DSTATE], sC[SSD_MAX_DSTATE];
  const int h = blockIdx.x, b = blockIdx.y;
  const int g = h / (H / G);
  const int tid = threadIdx.x;
  const int pv = P / 4;                 // f32x4 columns per row
  const int nr = kThreads / pv;         // rows processed per pass
  const int r = tid / pv, q = tid % pv;

  for (int n = tid; n < N; n += kThreads) {
    sB[n] = to_f32(B[(size_t(b) * G + g) * N + n]);
    sC[n] = to_f32(C[(size_t(b) * G + g) * N + n]);
  }
  const float d = to_f32(dt[size_t(b) * H + h]);
  const float a = expf(d * A[h]);
  f32x4 xv = f32x4{0.f, 0.f, 0.f, 0.f};
  const size_t xrow = (size_t(b) * H + h) * P;
  if (r < nr) {
    xv.x = to_f32(x[xrow + 4 * q + 0]);
    xv.y = to_f32(x[xrow + 4 * q + 1]);
    xv.z = to_f32(x[xrow + 4 * q + 2]);
    xv.w = to_f32(x[xrow + 4 * q + 3]);
  }
  __syncthreads();

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (r < nr) {
    float* st = state + (size_t(b) * H + h) * size_t(N) * P + 4 * q;
    for (int n = r; n < N; n += nr) {
      f32x4* p4 = reinterpret_cast<f32x4*>(st + size_t(n) * P);
      f32x4 hv = __builtin_nontemporal_load(p4);
      const float bb = d * sB[n];
      hv.x = a * hv.x + bb * xv.x;
      hv.y = a * hv.y + bb * xv.y;
      hv.z = a * hv.z + bb * xv.z;
      hv.w = a * hv.w + bb * xv.w;
      __builtin_nontemporal_store(hv, p4);
      const float cc = sC[n];
      acc.x += cc * hv.x;
      acc.y += cc * hv.y;
      acc.z += cc * hv.z;
      acc.w += cc * hv.w;
    }
  }
  part[tid] = acc;
  __syncthreads();
  if (tid < pv) {
    f32x4 s = part[tid];
    for (int rr = 1; rr < nr; ++rr) {
      const f32x4 o = part[rr * pv + tid];
      s.x += o.x; s.y += o.y; s.z += o.z; s.w += o.w;
    }
    const float Dh = D ? D[h] : 0.f;
    y[xrow + 4 * tid + 0] = from_f32<In>(s.x + Dh * xv.x);
    y[xrow + 4 * tid + 1] = from_f32<In>(s.y + Dh * xv.y);
    y[xrow + 4 * tid + 2] = from_f32<In>(s.z + Dh * xv.z);
    y[xrow + 4 * tid + 3] = from_f32<In>(s.w + Dh * xv.w);
  }
}

// Any headdim: one column per thread.
template <typename In>
__global__ __launch_bounds__(kThreads) void state_update_scalar(
    float* __restrict__ state, const In* __restrict__ x, const In* __restrict__ dt,
    const float* __restrict__ A, const In* __restrict__ B, const In* __restrict__ C,
    const float* __restrict__ D, In* __restrict__ y, int H, int P, int N, int G) {
  __shared__ float part[kThreads];
  const int h = blockIdx.x, b = blockIdx.y;
  const int g = h / (H / G);
  const int tid = threadIdx.x;
  const int nr = kThreads / P;
  const int r = tid / P, p = tid % P;
  const float d = to_f32(dt[size_t(b) * H + h]);
  const float a = expf(d * A[h]);
  const size_t xrow = (size_t(b) * H + h) * P;
  const float xp = r < nr ? to_f32(x[xrow + p]) : 0.f;
  float acc = 0.f;
  if (r < nr) {
    for (int n = r; n < N; n += nr) {
      const size_t si = ((size_t(b) * H + h) * N + n) * P + p;
      const float hn = a * state[si] + (d * to_f32(B[(size_t(b) * G + g) * N + n])) * xp;
      state[si] = hn;
      acc += to_f32(C[(size_t(b) * G + g) * N + n]) * hn;
    }
  }
  part[tid] = acc;
  __syncthreads();
  if (tid < P) {
    float s = 0.f;
    for (int rr = 0; rr < nr; ++rr) s += part[rr * P + tid];
    y[xrow + tid] = from_f32<In>(s + (D ? D[h] : 0.f) * xp);
  }
}

}  // namespace

hipError_t launch_state_update(ssd_dtype type, float* state, const void* x, const void* dt,
                               const float* A, const void* B, const void* C, const float* D, void* y,
                               int batch, int H, int P, int N, int G, hipStream_t st) {
  dim3 grid(H, batch);
  const bool vec = (P % 4 == 0);
  if (type == SSD_BF16) {
    auto k = vec ? state_update_vec4<uint16_t> : state_update_scalar<uint16_t>;
    hipLaunchKernelGGL(k, grid, dim3(kThreads), 0, st, state, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(dt), A, static_cast<const uint16_t*>(B),
                       static_cast<const uint16_t*>(C), D, static_cast<uint16_t*>(y), H, P, N, G);
  } else {
    auto k = vec ? state_update_vec4<float> : state_update_scalar<float>;
    hipLaunchKernelGGL(k, grid, dim3(kThreads), 0, st, state, static_cast<const float*>(x),
                       static_cast<const float*>(dt), A, static_cast<const float*>(B),
                       static_cast<const float*>(C), D, static_cast<float*>(y), H, P, N, G);
  }
  return hipGetLastError();
}

}  // namespace ssd
