// state_passing.hip -- the inter-chunk recurrence of the chunked algorithm.
//
//   H_0 = init (or 0);  for c = 0 .. nc-1:  out_c = H_c;  H_{c+1} = exp(Acs_c[Q-1]) H_c + S_c
//   final = H_nc
//
// out_c, the state entering chunk c, is what chunk_scan reads. This is the
// "state passed between chunks by the SSM recurrence" step (youngju.dev
// "Mamba / selective SSM", section "SSDアルゴリズムとチャンク分割"; Qiita
// "Mamba-2" article, section 4.2, step 3: scan across chunks).
// exp(Acs_c[Q-1]) is the decay of a whole chunk, the product of its abar_t.
//
// Chunk states are stored transposed ([p][n], n fastest); init_state and
// final_state use the caller's [n][p] layout, so the work-group that owns a
// 16 (p) x 64 (n) tile of one (b, h) state transposes them through LDS.
// The running state stays fp32. out_c goes either back over S_c (fp32, the
// generic path) or to a separate bf16 buffer (the MFMA path, whose chunk_scan
// consumes it as a bf16 matrix operand).
//
// Packed variable-length sequences run the same recurrence once per
// sequence, over that sequence's own chunk slots, from its initial state (or
// zero), and its last state is its final state (youngju.dev page, section on
// state initialisation and sequence boundaries: no state crosses from one
// sequence into the next); a sequence without tokens passes its initial
// state through.
//
// Elementwise and HBM-bound: each thread owns 4 consecutive n of one p and
// walks the chunks in order. Chunk states of later chunks do not depend on
// the recurrence, so their loads are issued kDepth chunks ahead of use.
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kDepth = 8;   // chunks of S in flight per thread
constexpr int kTP = 16;     // p rows per tile
constexpr int kTN = 64;     // n columns per tile (16 threads x 4)

// out_c: fp32 over S at idx ([p][n] rows), or bf16 to Hb at hidx (the
// fragment order of hb_off; 4 consecutive n stay consecutive there)
__device__ __forceinline__ void store_out(float* S, uint16_t* Hb, size_t idx, size_t hidx, const f32x4& v) {
  if (Hb) {
    const uint32_t lo = f32x2_to_bf16x2(v.x, v.y);
    const uint32_t hi = f32x2_to_bf16x2(v.z, v.w);
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<u32x2*>(Hb + hidx) = u32x2{lo, hi};
  } else {
    *reinterpret_cast<f32x4*>(S + idx) = v;
  }
}

// grid: b * H * ceil(P/kTP) * ceil(N/kTN) work-groups; requires N % 4 == 0.
// VARLEN: b counts sequences instead of batch rows, and the chunks of
// sequence b are its slots of the one packed row (cu: sequence offsets, T:
// packed tokens); init / fin are [nseq, H, N, P] like a batch of nseq rows.
template <bool VARLEN>
__global__ __launch_bounds__(kThreads) void state_passing_tiled(
    float* __restrict__ S, uint16_t* __restrict__ Hb, const float* __restrict__ Acs,
    const float* __restrict__ init, float* __restrict__ fin, int H, int P, int N, int Q, int nc,
    const int* __restrict__ cu, int T, int sfrag) {
  __shared__ float tile[kTN][kTP + 1];
  const int tpn = (N + kTN - 1) / kTN, tpp = (P + kTP - 1) / kTP;
  int bid = blockIdx.x;
  const int tn = bid % tpn; bid /= tpn;
  const int tp = bid % tpp; bid /= tpp;
  const int bh = bid;                       // b * H + h
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x;
  const int pi = tid / 16, nq = tid % 16;
  const int p0 = tp * kTP, n0 = tn * kTN;
  const int p = p0 + pi, n = n0 + 4 * nq;
  const bool active = p < P && n < N;
  const size_t sbh = size_t(N) * P;         // elements of one (b, h) state

  // the chunks this work-group walks: rows [crow, crow + ncw) of the chunk
  // arrays of batch row brow
  int brow = b, crow = 0, ncw = nc;
  if constexpr (VARLEN) {
    int s0, len;
    varlen_span(cu, b, T, s0, len);
    brow = 0;
    crow = varlen_first_slot(s0, b, Q);
    ncw = (len + Q - 1) / Q;
  }

  // H_0: init transposed through LDS (or zero)
  f32x4 cur = f32x4{0.f, 0.f, 0.f, 0.f};
  if (init) {
    for (int e = tid; e < kTN * kTP; e += kThreads) {
      const int nn = e / kTP, pp = e % kTP;
      float v = 0.f;
      if (n0 + nn < N && p0 + pp < P) v = init[size_t(bh) * sbh + size_t(n0 + nn) * P + p0 + pp];
      tile[nn][pp] = v;
    }
    __syncthreads();
    cur = f32x4{tile[4 * nq][pi], tile[4 * nq + 1][pi], tile[4 * nq + 2][pi], tile[4 * nq + 3][pi]};
    __syncthreads();
  }

  if (active) {
    const size_t cstride = size_t(H) * sbh;  // elements between chunk c and c+1
    // S in fragment order (sfrag: the segment states) or [p][n] rows
    const size_t off0 = ((size_t(brow) * nc + crow) * H + h) * sbh + (sfrag ? hb_off(p, n, N) : size_t(p) * N + n);
    // the same element of Hb (bf16 states, fragment order; needs P, N
    // multiples of 32, as the matrix-core path has)
    const size_t hoff0 = ((size_t(brow) * nc + crow) * H + h) * sbh + (Hb ? hb_off(p, n, N) : 0);
    const float* arow = Acs + ((size_t(brow) * H + h) * nc + crow) * Q + (Q - 1);
    f32x4 ring[kDepth];
    float dec[kDepth];
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      if (k < ncw) {
        ring[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + off0 + size_t(k) * cstride));
        dec[k] = arow[size_t(k) * Q];
      }
    }
    for (int c0 = 0; c0 < ncw; c0 += kDepth) {
#pragma unroll
      for (int k = 0; k < kDepth; ++k) {
        const int c = c0 + k;
        if (c < ncw) {
          const f32x4 s = ring[k];
          const float a = expf(dec[k]);
          if (c + kDepth < ncw) {
            ring[k] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4*>(S + off0 + size_t(c + kDepth) * cstride));
            dec[k] = arow[size_t(c + kDepth) * Q];
          }
          store_out(S, Hb, off0 + size_t(c) * cstride, hoff0 + size_t(c) * cstride, cur);
          cur.x = a * cur.x + s.x;
          cur.y = a * cur.y + s.y;
          cur.z = a * cur.z + s.z;
          cur.w = a * cur.w + s.w;
        }
      }
    }
  }

  // final state transposed back through LDS
  if (fin) {
    tile[4 * nq][pi] = cur.x;
    tile[4 * nq + 1][pi] = cur.y;
    tile[4 * nq + 2][pi] = cur.z;
    tile[4 * nq + 3][pi] = cur.w;
    __syncthreads();
    for (int e = tid; e < kTN * kTP; e += kThreads) {
      const int nn = e / kTP, pp = e % kTP;
      if (n0 + nn < N && p0 + pp < P) fin[size_t(bh) * sbh + size_t(n0 + nn) * P + p0 + pp] = tile[nn][pp];
    }
  }
}

// Any N (small shapes): one element per thread, fp32 in place.
__global__ __launch_bounds__(kThreads) void state_passing_scalar(
    float* __restrict__ S, const float* __restrict__ Acs, const float* __restrict__ init,
    float* __restrict__ fin, int H, int P, int N, int Q, int nc, long total) {
  const long i = long(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= total) return;
  const long bh = i / (long(N) * P);
  const int e = int(i % (long(N) * P));
  const int n = e / P, p = e % P;            // i walks the caller's [n][p] layout
  const int b = int(bh / H), h = int(bh % H);
  float cur = init ? init[i] : 0.f;
  for (int c = 0; c < nc; ++c) {
    const size_t si = ((size_t(b) * nc + c) * H + h) * size_t(N) * P + size_t(p) * N + n;
    const float s = S[si];
    S[si] = cur;
    cur = expf(Acs[(size_t(bh) * nc + c) * Q + Q - 1]) * cur + s;
  }
  if (fin) fin[i] = cur;
}

// Backward of the recurrence above. G_c, the gradient of the loss with
// respect to H_{c+1} (the state leaving chunk c), runs backwards:
//   G_{nc-1} = dfinal;  G_{c-1} = exp(Acs_c[Q-1]) G_c + dS_c;  dinit = G_{-1}
// where dS_c is what chunk c's outputs contribute to the gradient of the
// state entering it. Each G_c goes out as bf16, [p][n] like the chunk states,
// for the per-chunk gradient kernels, together with the partial sums
// of <G_c, H_c> (H_c the state entering chunk c: times exp(Acs_c[Q-1]), the
// part of the gradient of the chunk's total decay exponent that passes
// through H_c) of each wave of the work-group: ghp[b, c, h, tile, wave]. Hst
// holds the states entering each chunk (fp32, [p][n]). Same tiling as the
// forward kernel; dS, H_c and the decays of the chunks ahead (in reverse
// order) do not depend on the recurrence and are loaded kDepth chunks early.
__global__ __launch_bounds__(kThreads) void state_passing_bwd_tiled(
    const float* __restrict__ dS, const float* __restrict__ Hst,
    const float* __restrict__ Acs, const float* __restrict__ dfinal, uint16_t* __restrict__ Gb,
    float* __restrict__ ghp, float* __restrict__ dinit, int H, int P, int N, int Q, int nc) {
  __shared__ float tile[kTN][kTP + 1];
  const int tpn = (N + kTN - 1) / kTN, tpp = (P + kTP - 1) / kTP;
  int bid = blockIdx.x;
  const int tn = bid % tpn; bid /= tpn;
  const int tp = bid % tpp; bid /= tpp;
  const int bh = bid;
  const int b = bh / H, h = bh % H;
  const int tileid = tp * tpn + tn, ntiles = tpp * tpn;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pi = tid / 16, nq = tid % 16;
  const int p0 = tp * kTP, n0 = tn * kTN;
  const int p = p0 + pi, n = n0 + 4 * nq;
  const bool active = p < P && n < N;
  const size_t sbh = size_t(N) * P;

  // an [n][p] state of this (b, h), this thread's 4 elements, through LDS
  auto load_np = [&](const float* src) {
    for (int e = tid; e < kTN * kTP; e += kThreads) {
      const int nn = e / kTP, pp = e % kTP;
      float v = 0.f;
      if (src && n0 + nn < N && p0 + pp < P) v = src[size_t(bh) * sbh + size_t(n0 + nn) * P + p0 + pp];
      tile[nn][pp] = v;
    }
    __syncthreads();
    const f32x4 r = f32x4{tile[4 * nq][pi], tile[4 * nq + 1][pi], tile[4 * nq + 2][pi], tile[4 * nq + 3][pi]};
    __syncthreads();
    return r;
  };
  f32x4 G = load_np(dfinal);

  const size_t cstride = size_t(H) * sbh;
  const size_t off0 = (size_t(b) * nc * H + h) * sbh + size_t(p) * N + n;
  const float* arow = Acs + size_t(bh) * nc * Q + (Q - 1);
  // ring of the chunks ahead: slot k holds chunk nc-1-(m+k) for step m
  f32x4 rds[kDepth], rhc[kDepth];
  float rdec[kDepth];
  auto fetch = [&](int k, int c) {
    if (active) {
      const size_t o = off0 + size_t(c) * cstride;
      rds[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(dS + o));
      rhc[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Hst + o));
    } else {
      rds[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      rhc[k] = rds[k];
    }
    rdec[k] = arow[size_t(c) * Q];
  };
#pragma unroll
  for (int k = 0; k < kDepth; ++k)
    if (k < nc) fetch(k, nc - 1 - k);
  for (int m0 = 0; m0 < nc; m0 += kDepth) {
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      const int m = m0 + k;
      if (m < nc) {
        const int c = nc - 1 - m;
        const f32x4 ds = rds[k], hc = rhc[k];
        const float a = expf(rdec[k]);
        if (m + kDepth < nc) fetch(k, c - kDepth);
        if (active) store_out(nullptr, Gb, 0, off0 + size_t(c) * cstride, G);
        float dot = active ? G.x * hc.x + G.y * hc.y + G.z * hc.z + G.w * hc.w : 0.f;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
        if (lane == 0) ghp[((size_t(bh) * nc + c) * ntiles + tileid) * (kThreads / 64) + wave] = dot;
        G.x = a * G.x + ds.x;
        G.y = a * G.y + ds.y;
        G.z = a * G.z + ds.z;
        G.w = a * G.w + ds.w;
      }
    }
  }

  if (dinit) {
    tile[4 * nq][pi] = G.x;
    tile[4 * nq + 1][pi] = G.y;
    tile[4 * nq + 2][pi] = G.z;
    tile[4 * nq + 3][pi] = G.w;
    __syncthreads();
    for (int e = tid; e < kTN * kTP; e += kThreads) {
      const int nn = e / kTP, pp = e % kTP;
      if (n0 + nn < N && p0 + pp < P) dinit[size_t(bh) * sbh + size_t(n0 + nn) * P + p0 + pp] = tile[nn][pp];
    }
  }
}

// Packed sequences through the fused walk: the recurrence over segments
// (launch_varlen_segment_recurrence). Work-groups 0 .. ntiles-1: one (head,
// 16 x 64 tile) each, walking the segments in order with S and the decay
// exponents of the segments ahead loaded kDepth segments early (they do
// not depend on the recurrence); a final state completed at segment k (its F
// read then) goes out through LDS in the caller's [n][p] layout. Work-groups
// ntiles + i: an empty sequence i's final state is its initial state (or
// zero).
__global__ __launch_bounds__(kThreads) void varlen_segment_recurrence(
    float* __restrict__ S, const float* __restrict__ F, const float* __restrict__ segdec,
    const float* __restrict__ fdec, const int* __restrict__ fseq, const int* __restrict__ cu,
    const float* __restrict__ init, float* __restrict__ fin, int H, int P, int N, int nseg, int nseq, int T,
    int ntiles) {
  __shared__ float tile[kTN][kTP + 1];
  const int tid = threadIdx.x;
  const size_t sbh = size_t(N) * P;          // elements of one head's state
  if (int(blockIdx.x) >= ntiles) {
    const int i = int(blockIdx.x) - ntiles;   // < nseq by the grid
    int s0, len;
    varlen_span(cu, i, T, s0, len);
    if (len > 0 || !fin) return;
    const size_t base = size_t(i) * H * sbh;
    for (size_t e = tid; e < size_t(H) * sbh; e += kThreads) fin[base + e] = init ? init[base + e] : 0.f;
    return;
  }
  const int tpn = (N + kTN - 1) / kTN, tpp = (P + kTP - 1) / kTP;
  int bid = blockIdx.x;
  const int tn = bid % tpn; bid /= tpn;
  const int tp = bid % tpp; bid /= tpp;
  const int h = bid;                         // < H by the grid
  const int pi = tid / 16, nq = tid % 16;
  const int p0 = tp * kTP, n0 = tn * kTN;
  const int p = p0 + pi, n = n0 + 4 * nq;    // P, N multiples of 32: every thread active
  const size_t cstride = size_t(H) * sbh;    // elements between segment k and k + 1
  const size_t off0 = size_t(h) * sbh + hb_off(p, n, N);
  const float* sd = segdec + size_t(h) * nseg;
  const float* fd = fdec + size_t(h) * nseg;
  f32x4 rs[kDepth], rf[kDepth];
  float rsd[kDepth], rfd[kDepth];
  int rfs[kDepth];
  // F (the local end state of a sequence that ends in segment k) is fetched
  // with S, used only where fseq[k] names such a sequence: a load and its
  // wait per ending would otherwise sit on the chain
  auto fetch = [&](int k, int j) {
    rs[j] = *reinterpret_cast<const f32x4*>(S + off0 + size_t(k) * cstride);
    rf[j] = *reinterpret_cast<const f32x4*>(F + off0 + size_t(k) * cstride);
    rsd[j] = sd[k];
    rfd[j] = fd[k];
    rfs[j] = fseq[k];
  };
#pragma unroll
  for (int j = 0; j < kDepth; ++j)
    if (j < nseg) fetch(j, j);
  f32x4 carry = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < nseg; k0 += kDepth) {
#pragma unroll
    for (int j = 0; j < kDepth; ++j) {
      const int k = k0 + j;
      if (k < nseg) {
        const f32x4 e = rs[j], fk = rf[j];
        const float a = expf(rsd[j]), af = expf(rfd[j]);
        const int fs = rfs[j];                 // uniform
        if (k + kDepth < nseg) fetch(k + kDepth, j);
        if (fs >= 0 && fs < nseq && fin) {
          // sequence fs, continued into segment k, ends there
          tile[4 * nq][pi] = fk.x + af * carry.x;
          tile[4 * nq + 1][pi] = fk.y + af * carry.y;
          tile[4 * nq + 2][pi] = fk.z + af * carry.z;
          tile[4 * nq + 3][pi] = fk.w + af * carry.w;
          __syncthreads();
          for (int q = tid; q < kTN * kTP; q += kThreads) {
            const int nn = q / kTP, pp = q % kTP;
            fin[(size_t(fs) * H + h) * sbh + size_t(n0 + nn) * P + p0 + pp] = tile[nn][pp];
          }
          __syncthreads();
        }
        *reinterpret_cast<f32x4*>(S + off0 + size_t(k) * cstride) = carry;   // the state entering segment k
        carry.x = a * carry.x + e.x;
        carry.y = a * carry.y + e.y;
        carry.z = a * carry.z + e.z;
        carry.w = a * carry.w + e.w;
      }
    }
  }
}

}  // namespace

int state_passing_bwd_partials(const FwdShape& s) {
  return ((s.P + kTP - 1) / kTP) * ((s.N + kTN - 1) / kTN) * (kThreads / 64);
}

hipError_t launch_state_passing_bwd(const FwdShape& s, const float* dS, const float* Hst, const float* Acs,
                                    const float* dfinal, uint16_t* Gb, float* ghp, float* dinit, hipStream_t st) {
  if (s.N % 4) return hipErrorInvalidValue;
  const long tiles = long(s.b) * s.H * ((s.P + kTP - 1) / kTP) * ((s.N + kTN - 1) / kTN);
  hipLaunchKernelGGL(state_passing_bwd_tiled, dim3(unsigned(tiles)), dim3(kThreads), 0, st, dS, Hst, Acs,
                     dfinal, Gb, ghp, dinit, s.H, s.P, s.N, s.Q, s.nc);
  return hipGetLastError();
}

hipError_t launch_state_passing_varlen(const FwdShape& s, const float* S, uint16_t* Hb, const float* Acs,
                                       const int* cu, int nseq, const float* init, float* final_state,
                                       hipStream_t st, const StageEv& ev) {
  if (s.N % 4 || !Hb) return hipErrorInvalidValue;   // matrix-core path only
  const long tiles = long(nseq) * s.H * ((s.P + kTP - 1) / kTP) * ((s.N + kTN - 1) / kTN);
  // S is only read: the passed states go to Hb
  hipExtLaunchKernelGGL(state_passing_tiled<true>, dim3(unsigned(tiles)), dim3(kThreads), 0, st, ev.start,
                        ev.stop, 0, const_cast<float*>(S), Hb, Acs, init, final_state, s.H, s.P, s.N, s.Q,
                        s.nc, cu, s.T, 0);
  return hipGetLastError();
}

hipError_t launch_varlen_segment_recurrence(const FwdShape& s, float* S, const float* F, const float* segdec,
                                            const float* fdec, const int* fseq, const int* cu, int nseq,
                                            const float* init, float* final_state, hipStream_t st,
                                            const StageEv& ev) {
  if (s.N % 32 || s.P % 32 || s.b != 1 || s.nc < 1 || nseq < 1) return hipErrorInvalidValue;
  const long tiles = long(s.H) * ((s.P + kTP - 1) / kTP) * ((s.N + kTN - 1) / kTN);
  hipExtLaunchKernelGGL(varlen_segment_recurrence, dim3(unsigned(tiles + nseq)), dim3(kThreads), 0, st, ev.start,
                        ev.stop, 0, S, F, segdec, fdec, fseq, cu, init, final_state, s.H, s.P, s.N, s.nc, nseq,
                        s.T, int(tiles));
  return hipGetLastError();
}

hipError_t launch_state_passing(const FwdShape& s, float* S, uint16_t* Hb, const float* Acs,
                                const float* init, float* final_state, hipStream_t st, const StageEv& ev,
                                bool sfrag) {
  if (sfrag && (s.N % 32 || s.P % 32)) return hipErrorInvalidValue;
  if (s.N % 4 == 0) {
    const long tiles = long(s.b) * s.H * ((s.P + kTP - 1) / kTP) * ((s.N + kTN - 1) / kTN);
    hipExtLaunchKernelGGL(state_passing_tiled<false>, dim3(unsigned(tiles)), dim3(kThreads), 0, st, ev.start,
                          ev.stop, 0, S, Hb, Acs, init, final_state, s.H, s.P, s.N, s.Q, s.nc,
                          static_cast<const int*>(nullptr), 0, sfrag ? 1 : 0);
  } else {
    if (Hb) return hipErrorInvalidValue;     // the MFMA path never has N % 4 != 0
    const long total = long(s.b) * s.H * s.N * s.P;
    const long blocks = (total + kThreads - 1) / kThreads;
    hipExtLaunchKernelGGL(state_passing_scalar, dim3(unsigned(blocks)), dim3(kThreads), 0, st, ev.start, ev.stop, 0, S, Acs,
                       init, final_state, s.H, s.P, s.N, s.Q, s.nc, total);
  }
  return hipGetLastError();
}

}  // namespace ssd
