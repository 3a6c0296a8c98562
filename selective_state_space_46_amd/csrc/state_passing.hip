// state_passing.hip -- the inter-chunk recurrence of the chunked algorithm.
//
//   H_0 = init (or 0);  for c = 0 .. nc-1:  out_c = H_c;  H_{c+1} = exp(Acs_c[Q-1]) H_c + S_c
//   final = H_nc
//
// Chunk c's own state S_c (from chunk_state) is replaced in place by H_c, the
// state entering chunk c, which chunk_scan reads. This is the "state passed
// between chunks by the SSM recurrence" step (youngju.dev "Mamba / selective
// SSM", section "SSDアルゴリズムとチャンク分割"; Qiita "Mamba-2" article,
// section 4.2, step 3: scan across chunks). exp(Acs_c[Q-1]) is the decay of a
// whole chunk, the product of its abar_t.
//
// Elementwise and HBM-bound: each thread owns 4 consecutive fp32 elements of
// one (b, h) state and walks the chunks sequentially. The chunk states of
// later chunks do not depend on the recurrence, so their loads are issued
// kDepth chunks ahead of use to keep enough bytes in flight.
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kDepth = 8;  // chunks of S in flight per thread

__global__ __launch_bounds__(kThreads) void state_passing_kernel(
    float* __restrict__ S, const float* __restrict__ Acs, const float* __restrict__ init,
    float* __restrict__ fin, int H, int NP, int Q, int nc, long nvec /* b*H*NP/4 */) {
  const long v = long(blockIdx.x) * kThreads + threadIdx.x;
  if (v >= nvec) return;
  const int nvh = NP / 4;                  // f32x4 per (b,h) state
  const long bh = v / nvh;
  const int e = int(v % nvh) * 4;
  const int b = int(bh / H), h = int(bh % H);
  const size_t cstride = size_t(H) * NP;   // elements between chunk c and c+1
  float* base = S + (size_t(b) * nc * H + h) * NP + e;
  const float* arow = Acs + size_t(bh) * nc * Q + (Q - 1);

  f32x4 cur = f32x4{0.f, 0.f, 0.f, 0.f};
  if (init) cur = *reinterpret_cast<const f32x4*>(init + size_t(bh) * NP + e);

  f32x4 ring[kDepth];
  float dec[kDepth];
#pragma unroll
  for (int k = 0; k < kDepth; ++k) {
    if (k < nc) {
      ring[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(base + size_t(k) * cstride));
      dec[k] = arow[size_t(k) * Q];
    }
  }
  for (int c0 = 0; c0 < nc; c0 += kDepth) {
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      const int c = c0 + k;
      if (c < nc) {
        const f32x4 s = ring[k];
        const float a = expf(dec[k]);
        if (c + kDepth < nc) {
          ring[k] = __builtin_nontemporal_load(
              reinterpret_cast<const f32x4*>(base + size_t(c + kDepth) * cstride));
          dec[k] = arow[size_t(c + kDepth) * Q];
        }
        *reinterpret_cast<f32x4*>(base + size_t(c) * cstride) = cur;
        cur.x = a * cur.x + s.x;
        cur.y = a * cur.y + s.y;
        cur.z = a * cur.z + s.z;
        cur.w = a * cur.w + s.w;
      }
    }
  }
  if (fin) *reinterpret_cast<f32x4*>(fin + size_t(bh) * NP + e) = cur;
}

// Scalar variant for N*P not a multiple of 4.
__global__ __launch_bounds__(kThreads) void state_passing_scalar(
    float* __restrict__ S, const float* __restrict__ Acs, const float* __restrict__ init,
    float* __restrict__ fin, int H, int NP, int Q, int nc, long total) {
  const long i = long(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= total) return;
  const long bh = i / NP;
  const int e = int(i % NP);
  const int b = int(bh / H), h = int(bh % H);
  float cur = init ? init[i] : 0.f;
  for (int c = 0; c < nc; ++c) {
    const size_t si = ((size_t(b) * nc + c) * H + h) * NP + e;
    const float s = S[si];
    S[si] = cur;
    cur = expf(Acs[(size_t(bh) * nc + c) * Q + Q - 1]) * cur + s;
  }
  if (fin) fin[i] = cur;
}

}  // namespace

hipError_t launch_state_passing(const FwdShape& s, float* S, const float* Acs, const float* init,
                                float* final_state, hipStream_t st) {
  const int NP = s.N * s.P;
  if (NP % 4 == 0) {
    const long nvec = long(s.b) * s.H * NP / 4;
    const long blocks = (nvec + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(state_passing_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, st, S, Acs,
                       init, final_state, s.H, NP, s.Q, s.nc, nvec);
  } else {
    const long total = long(s.b) * s.H * NP;
    const long blocks = (total + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(state_passing_scalar, dim3(unsigned(blocks)), dim3(kThreads), 0, st, S, Acs,
                       init, final_state, s.H, NP, s.Q, s.nc, total);
  }
  return hipGetLastError();
}

}  // namespace ssd
