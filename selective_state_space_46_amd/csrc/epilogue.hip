// epilogue.hip -- the two element-wise stages next to the SSD core.
//
// Gated RMS normalisation (after the core): the SSD output y is RMS-normalised
// and gated by SiLU of the gate branch z, rmsnorm(y) * silu(z) (Qiita "Mamba-2"
// article, section 4.2, SSD block step 4):
//   out[t, c] = y[t, c] * rsqrt(mean_{c' in group(c)} y[t, c']^2 + eps) * w[c] * silu(z[t, c])
// over groups of `group` consecutive channels of each token's feature vector
// (the whole vector, or one head), silu(z) = z / (1 + exp(-z)).
//
// Depthwise causal convolution (before the core): the Mamba block's
// Conv1d(d, d, K, padding K-1, groups d, bias) trimmed to the first L outputs,
// then SiLU (youngju.dev "Mamba / selective SSM" page, the Mamba block code):
//   out[t, c] = act(bias[c] + sum_{k<K} w[c, k] x[t - (K-1) + k, c])
// with the K-1 tokens before token 0 taken from a carried state (zeros when
// absent), channels-last [b, T, C]; its one-token recurrent form updates a
// [b, K-1, C] state in place (decode).
//
// All of them are HBM-bound streams: each element is read once and written
// once (the convolution's K-1 token halo and the norm's second pass come from
// registers or L1/L2).
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kConvTok = 16;   // tokens per thread in the convolution

template <typename T> struct Vec;       // elements per 16-byte vector
template <> struct Vec<uint16_t> { static constexpr int n = 8; };
template <> struct Vec<float> { static constexpr int n = 4; };

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float silu_f(float z) {
  // z / (1 + e^-z), e^-z = 2^(-z log2 e); for very negative z the
  // exponential is +inf and the result is -0
  return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

__device__ __forceinline__ float to_float(uint16_t v) { return bf16_to_f32(v); }
__device__ __forceinline__ float to_float(float v) { return v; }
template <typename T> __device__ __forceinline__ T from_float(float f);
template <> __device__ __forceinline__ uint16_t from_float<uint16_t>(float f) { return f32_to_bf16(f); }
template <> __device__ __forceinline__ float from_float<float>(float f) { return f; }

// one 16-byte vector <-> Vec<T>::n floats
template <typename T>
__device__ __forceinline__ void unpack(const u32x4_t& v, float (&f)[Vec<T>::n]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
}
template <typename T>
__device__ __forceinline__ u32x4_t pack(const float (&f)[Vec<T>::n]) {
  u32x4_t v;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = f32x2_to_bf16x2(f[2 * i], f[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ---------------------------------------------------------------------------
// Gated RMS normalisation. Row r = (token, group) is `group` contiguous
// channels at r * group; its weights start at (r % groups_per_token) * group.
// out may be y itself (each element is read before the same lane writes it),
// so y carries no restrict qualifier.

// vector path (group % VEC == 0): one wave per row, lane vectors at
// (step * 64 + lane) * VEC; the row stays in registers between the two passes
template <typename T, int STEPS>
__global__ __launch_bounds__(kThreads) void gated_rmsnorm_vec(const T* y,
                                                              const T* __restrict__ z,
                                                              const float* __restrict__ w,
                                                              T* out, long nrows, int group,
                                                              int gpt, float eps) {
  constexpr int VEC = Vec<T>::n;
  const long row = long(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= nrows) return;                     // wave-uniform; no barriers here
  const int lane = threadIdx.x & 63;
  const size_t base = size_t(row) * group;
  const float* wr = w + size_t(row % gpt) * group;
  const int nvec = group / VEC;
  u32x4_t yv[STEPS];
  float ss = 0.f;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int v = s * 64 + lane;
    yv[s] = v < nvec ? *reinterpret_cast<const u32x4_t*>(y + base + size_t(v) * VEC) : u32x4_t{0u, 0u, 0u, 0u};
    float f[VEC];
    unpack<T>(yv[s], f);
#pragma unroll
    for (int i = 0; i < VEC; ++i) ss += f[i] * f[i];
  }
  const float rinv = rsqrtf(wave_sum(ss) / float(group) + eps);
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int v = s * 64 + lane;
    if (v < nvec) {
      float fy[VEC], fz[VEC], o[VEC];
      unpack<T>(yv[s], fy);
      unpack<T>(*reinterpret_cast<const u32x4_t*>(z + base + size_t(v) * VEC), fz);
#pragma unroll
      for (int i = 0; i < VEC; ++i) o[i] = fy[i] * rinv * wr[v * VEC + i] * silu_f(fz[i]);
      *reinterpret_cast<u32x4_t*>(out + base + size_t(v) * VEC) = pack<T>(o);
    }
  }
}

// any group: one wave per row, lane-strided elements, two passes over memory
template <typename T>
__global__ __launch_bounds__(kThreads) void gated_rmsnorm_scalar(const T* y,
                                                                 const T* __restrict__ z,
                                                                 const float* __restrict__ w,
                                                                 T* out, long nrows, int group,
                                                                 int gpt, float eps) {
  const long row = long(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= nrows) return;
  const int lane = threadIdx.x & 63;
  const size_t base = size_t(row) * group;
  const float* wr = w + size_t(row % gpt) * group;
  float ss = 0.f;
  for (int c = lane; c < group; c += 64) {
    const float f = to_float(y[base + c]);
    ss += f * f;
  }
  const float rinv = rsqrtf(wave_sum(ss) / float(group) + eps);
  for (int c = lane; c < group; c += 64)
    out[base + c] = from_float<T>(to_float(y[base + c]) * rinv * wr[c] * silu_f(to_float(z[base + c])));
}

// ---------------------------------------------------------------------------
// Depthwise causal convolution. Thread per (batch, run of kConvTok tokens, V
// channels) with V = 4 on the vector path (C % 4 == 0: 8-byte bf16 or 16-byte
// fp32 accesses) and V = 1 otherwise. The K-1 tokens before the run come from
// x (or from the carried state before token 0) and then slide through
// registers, so x is read once plus a K-1-token halo per run; on a full run
// all token loads are issued before the first use (one memory latency per
// run, not per token).
template <typename T, int V> struct Chunk;          // V elements of T in one access
template <> struct Chunk<uint16_t, 4> { typedef uint32_t raw __attribute__((ext_vector_type(2))); };
template <> struct Chunk<float, 4> { typedef uint32_t raw __attribute__((ext_vector_type(4))); };
template <typename T> struct Chunk<T, 1> { typedef T raw; };

template <typename T, int V>
__device__ __forceinline__ void chunk_to_f(const typename Chunk<T, V>::raw& r, float (&f)[V]) {
  if constexpr (V == 1) {
    f[0] = to_float(r);
  } else if constexpr (sizeof(T) == 2) {
    f[0] = __uint_as_float(r[0] << 16);
    f[1] = __uint_as_float(r[0] & 0xffff0000u);
    f[2] = __uint_as_float(r[1] << 16);
    f[3] = __uint_as_float(r[1] & 0xffff0000u);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(r[i]);
  }
}
template <typename T, int V>
__device__ __forceinline__ typename Chunk<T, V>::raw f_to_chunk(const float (&f)[V]) {
  typename Chunk<T, V>::raw r;
  if constexpr (V == 1) {
    r = from_float<T>(f[0]);
  } else if constexpr (sizeof(T) == 2) {
    r[0] = f32x2_to_bf16x2(f[0], f[1]);
    r[1] = f32x2_to_bf16x2(f[2], f[3]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(f[i]);
  }
  return r;
}

// fin (or null): the final state, written by the thread of each column's
// last run from its window (the last K-1 values of carried state and x).
// Only passed when no other thread still reads the carried state it may
// overwrite: fin is not the carried state, or a row is one run.
template <typename T, int K, int V>
__global__ __launch_bounds__(kThreads) void conv1d_fwd(const T* __restrict__ x,
                                                       const float* __restrict__ w,
                                                       const float* __restrict__ bias,
                                                       const T* init, T* __restrict__ out, T* fin,
                                                       int b_, int T_, int C, int nruns, int act) {
  typedef typename Chunk<T, V>::raw raw_t;
  const int nv = C / V;
  const long total = long(b_) * nruns * nv;
  const long gid = long(blockIdx.x) * kThreads + threadIdx.x;
  if (gid >= total) return;                     // no barriers in this kernel
  const int cv = int(gid % nv);
  const long br = gid / nv;
  const int run = int(br % nruns), b = int(br / nruns);
  const int c0 = cv * V;
  float wk[K][V], bv[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    bv[i] = bias ? bias[c0 + i] : 0.f;
    if constexpr (K == 4) {            // one 16-byte load per channel (weight rows are 16-byte aligned)
      const f32x4 wv = *reinterpret_cast<const f32x4*>(w + size_t(c0 + i) * 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) wk[k][i] = wv[k];
    } else {
#pragma unroll
      for (int k = 0; k < K; ++k) wk[k][i] = w[size_t(c0 + i) * K + k];
    }
  }
  const int t0 = run * kConvTok;
  const T* xb = x + size_t(b) * T_ * C + c0;
  T* ob = out + size_t(b) * T_ * C + c0;
  auto ld = [&](const T* p) { return *reinterpret_cast<const raw_t*>(p); };
  // win[k] holds token t - (K-1) + k for the next output t
  float win[K][V];
#pragma unroll
  for (int k = 0; k < K - 1; ++k) {
    const int t = t0 - (K - 1) + k;
    if (t >= 0) {
      chunk_to_f<T, V>(ld(xb + size_t(t) * C), win[k]);
    } else if (init) {
      chunk_to_f<T, V>(ld(init + (size_t(b) * (K - 1) + (t + K - 1)) * C + c0), win[k]);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) win[k][i] = 0.f;
    }
  }
  // one output token from the window (win[K-1] just filled), then slide
  auto step = [&](int t) {
    float o[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float a = bv[i];
#pragma unroll
      for (int k = 0; k < K; ++k) a += wk[k][i] * win[k][i];
      o[i] = act ? silu_f(a) : a;
    }
    *reinterpret_cast<raw_t*>(ob + size_t(t) * C) = f_to_chunk<T, V>(o);
#pragma unroll
    for (int k = 0; k < K - 1; ++k)
#pragma unroll
      for (int i = 0; i < V; ++i) win[k][i] = win[k + 1][i];
  };
  if (t0 + kConvTok <= T_) {
    raw_t r[kConvTok];
#pragma unroll
    for (int j = 0; j < kConvTok; ++j) r[j] = ld(xb + size_t(t0 + j) * C);
#pragma unroll
    for (int j = 0; j < kConvTok; ++j) {
      chunk_to_f<T, V>(r[j], win[K - 1]);
      step(t0 + j);
    }
  } else {
    for (int t = t0; t < T_; ++t) {
      chunk_to_f<T, V>(ld(xb + size_t(t) * C), win[K - 1]);
      step(t);
    }
  }
  // after the last token win[0 .. K-2] holds the last K-1 values of (carried
  // state, x); bf16 -> fp32 -> bf16 is exact
  if (fin && run == nruns - 1) {
#pragma unroll
    for (int k = 0; k < K - 1; ++k)
      *reinterpret_cast<raw_t*>(fin + (size_t(b) * (K - 1) + k) * C + c0) = f_to_chunk<T, V>(win[k]);
  }
}

// final state: the last K-1 tokens of (carried state, x), one thread per
// (batch, channel) column; the column is read completely before it is
// written, so the final state may be the same buffer as the carried one
template <typename T, int K>
__global__ __launch_bounds__(kThreads) void conv1d_final(const T* __restrict__ x, const T* init,
                                                         T* fin, int b_, int T_, int C) {
  const long gid = long(blockIdx.x) * kThreads + threadIdx.x;
  if (gid >= long(b_) * C) return;
  const int c = int(gid % C), b = int(gid / C);
  T col[K > 1 ? K - 1 : 1];
#pragma unroll
  for (int k = 0; k < K - 1; ++k) {
    const int t = T_ - (K - 1) + k;             // token index in x; < 0: from the carried state
    if (t >= 0) col[k] = x[(size_t(b) * T_ + t) * C + c];
    else col[k] = init ? init[(size_t(b) * (K - 1) + (t + K - 1)) * C + c] : from_float<T>(0.f);
  }
#pragma unroll
  for (int k = 0; k < K - 1; ++k) fin[(size_t(b) * (K - 1) + k) * C + c] = col[k];
}

// one token, recurrent form: thread per (batch, channel), state column in
// place (measured faster than 4-channel vectors per thread: more threads in
// flight for this short stream)
template <typename T, int K>
__global__ __launch_bounds__(kThreads) void conv1d_update(T* state, const T* __restrict__ x,
                                                          const float* __restrict__ w,
                                                          const float* __restrict__ bias,
                                                          T* __restrict__ out, int b_, int C, int act) {
  const long gid = long(blockIdx.x) * kThreads + threadIdx.x;
  if (gid >= long(b_) * C) return;
  const int c = int(gid % C), b = int(gid / C);
  float win[K];
#pragma unroll
  for (int k = 0; k < K - 1; ++k) win[k] = to_float(state[(size_t(b) * (K - 1) + k) * C + c]);
  const T xn = x[size_t(b) * C + c];
  win[K - 1] = to_float(xn);
  float a = bias ? bias[c] : 0.f;
#pragma unroll
  for (int k = 0; k < K; ++k) a += w[size_t(c) * K + k] * win[k];
  out[size_t(b) * C + c] = from_float<T>(act ? silu_f(a) : a);
#pragma unroll
  for (int k = 0; k + 1 < K - 1; ++k) state[(size_t(b) * (K - 1) + k) * C + c] = state[(size_t(b) * (K - 1) + k + 1) * C + c];
  if (K > 1) state[(size_t(b) * (K - 1) + K - 2) * C + c] = xn;
}

template <typename T, int STEPS>
hipError_t norm_steps(const void* y, const void* z, const float* w, void* out, long nrows, int group,
                      int gpt, float eps, hipStream_t st) {
  const long blocks = (nrows + kThreads / 64 - 1) / (kThreads / 64);
  hipLaunchKernelGGL((gated_rmsnorm_vec<T, STEPS>), dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                     static_cast<const T*>(y), static_cast<const T*>(z), w, static_cast<T*>(out), nrows,
                     group, gpt, eps);
  return hipGetLastError();
}

template <typename T>
hipError_t norm_t(const void* y, const void* z, const float* w, void* out, long ntok, int dim, int group,
                  float eps, hipStream_t st) {
  constexpr int VEC = Vec<T>::n;
  const int gpt = dim / group;
  const long nrows = ntok * gpt;
  if (group % VEC == 0) {
    const int steps = (group / VEC + 63) / 64;
    switch (steps) {
      case 1: return norm_steps<T, 1>(y, z, w, out, nrows, group, gpt, eps, st);
      case 2: return norm_steps<T, 2>(y, z, w, out, nrows, group, gpt, eps, st);
      case 3: return norm_steps<T, 3>(y, z, w, out, nrows, group, gpt, eps, st);
      case 4: return norm_steps<T, 4>(y, z, w, out, nrows, group, gpt, eps, st);
      default: break;                           // long rows: the two-pass kernel
    }
  }
  const long blocks = (nrows + kThreads / 64 - 1) / (kThreads / 64);
  hipLaunchKernelGGL((gated_rmsnorm_scalar<T>), dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                     static_cast<const T*>(y), static_cast<const T*>(z), w, static_cast<T*>(out), nrows,
                     group, gpt, eps);
  return hipGetLastError();
}

template <typename T, int K>
hipError_t conv_k(const void* x, const float* w, const float* bias, const void* init, void* out, void* fin,
                  int b, int T_, int C, int act, hipStream_t st) {
  const int nruns = (T_ + kConvTok - 1) / kConvTok;
  const bool vec = C % 4 == 0;
  const long total = long(b) * nruns * (vec ? C / 4 : C);
  const long blocks = (total + kThreads - 1) / kThreads;
  // the final state from the main kernel where that cannot race with a read
  // of the carried state (see conv1d_fwd), else from a launch after it
  const bool fused = fin && K > 1 && (fin != init || nruns == 1);
  T* kfin = fused ? static_cast<T*>(fin) : nullptr;
  if (vec)
    hipLaunchKernelGGL((conv1d_fwd<T, K, 4>), dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                       static_cast<const T*>(x), w, bias, static_cast<const T*>(init), static_cast<T*>(out),
                       kfin, b, T_, C, nruns, act);
  else
    hipLaunchKernelGGL((conv1d_fwd<T, K, 1>), dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                       static_cast<const T*>(x), w, bias, static_cast<const T*>(init), static_cast<T*>(out),
                       kfin, b, T_, C, nruns, act);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  if (fin && K > 1 && !fused) {
    // after the main kernel in stream order: it has finished reading the
    // carried state, which the final state may overwrite
    const long fb = (long(b) * C + kThreads - 1) / kThreads;
    hipLaunchKernelGGL((conv1d_final<T, K>), dim3(unsigned(fb)), dim3(kThreads), 0, st,
                       static_cast<const T*>(x), static_cast<const T*>(init), static_cast<T*>(fin), b, T_, C);
  }
  return hipGetLastError();
}

template <typename T, int K>
hipError_t upd_k(void* state, const void* x, const float* w, const float* bias, void* out, int b, int C,
                 int act, hipStream_t st) {
  const long blocks = (long(b) * C + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((conv1d_update<T, K>), dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                     static_cast<T*>(state), static_cast<const T*>(x), w, bias, static_cast<T*>(out), b, C,
                     act);
  return hipGetLastError();
}

template <typename T>
hipError_t conv_t(const void* x, const float* w, const float* bias, const void* init, void* out, void* fin,
                  int b, int T_, int C, int K, int act, hipStream_t st) {
  switch (K) {
    case 1: return conv_k<T, 1>(x, w, bias, init, out, fin, b, T_, C, act, st);
    case 2: return conv_k<T, 2>(x, w, bias, init, out, fin, b, T_, C, act, st);
    case 3: return conv_k<T, 3>(x, w, bias, init, out, fin, b, T_, C, act, st);
    case 4: return conv_k<T, 4>(x, w, bias, init, out, fin, b, T_, C, act, st);
    case 5: return conv_k<T, 5>(x, w, bias, init, out, fin, b, T_, C, act, st);
    case 6: return conv_k<T, 6>(x, w, bias, init, out, fin, b, T_, C, act, st);
    case 7: return conv_k<T, 7>(x, w, bias, init, out, fin, b, T_, C, act, st);
    case 8: return conv_k<T, 8>(x, w, bias, init, out, fin, b, T_, C, act, st);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t upd_t(void* state, const void* x, const float* w, const float* bias, void* out, int b, int C, int K,
                 int act, hipStream_t st) {
  switch (K) {
    case 1: return upd_k<T, 1>(state, x, w, bias, out, b, C, act, st);
    case 2: return upd_k<T, 2>(state, x, w, bias, out, b, C, act, st);
    case 3: return upd_k<T, 3>(state, x, w, bias, out, b, C, act, st);
    case 4: return upd_k<T, 4>(state, x, w, bias, out, b, C, act, st);
    case 5: return upd_k<T, 5>(state, x, w, bias, out, b, C, act, st);
    case 6: return upd_k<T, 6>(state, x, w, bias, out, b, C, act, st);
    case 7: return upd_k<T, 7>(state, x, w, bias, out, b, C, act, st);
    case 8: return upd_k<T, 8>(state, x, w, bias, out, b, C, act, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gated_rmsnorm(ssd_dtype type, const void* y, const void* z, const float* w, void* out,
                                long ntok, int dim, int group, float eps, hipStream_t st) {
  return type == SSD_BF16 ? norm_t<uint16_t>(y, z, w, out, ntok, dim, group, eps, st)
                          : norm_t<float>(y, z, w, out, ntok, dim, group, eps, st);
}

hipError_t launch_causal_conv1d(ssd_dtype type, const void* x, const float* w, const float* bias,
                                const void* init, void* out, void* fin, int b, int T, int C, int K, int act,
                                hipStream_t st) {
  return type == SSD_BF16 ? conv_t<uint16_t>(x, w, bias, init, out, fin, b, T, C, K, act, st)
                          : conv_t<float>(x, w, bias, init, out, fin, b, T, C, K, act, st);
}

hipError_t launch_causal_conv1d_update(ssd_dtype type, void* state, const void* x, const float* w,
                                       const float* bias, void* out, int b, int C, int K, int act,
                                       hipStream_t st) {
  return type == SSD_BF16 ? upd_t<uint16_t>(state, x, w, bias, out, b, C, K, act, st)
                          : upd_t<float>(state, x, w, bias, out, b, C, K, act, st);
}

}  // namespace ssd
