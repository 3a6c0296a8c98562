// chunk_scan_mfma.hip -- chunk outputs on the bf16 matrix cores.
//
//   y_l = sum_{s <= l, same chunk} (C_l . B_s) exp(Acs_l - Acs_s) dt_s x_s
//       + exp(Acs_l) C_l^T H_c + D_h x_l
//
// The first term is the chunk's diagonal block of y = M x with the
// semiseparable M_ij = C_i^T abar_{i:j} B_j (youngju.dev "Mamba / selective
// SSM", section "State Space Dualityの発見"): the matrix C B^T, masked to the
// causal lower triangle and weighted by the decay, times dt*X -- the
// attention-like form with no softmax (Qiita "Mamba-2" article, section 3.3).
// The second term brings in all earlier chunks through H_c, the state entering
// chunk c (youngju.dev page, "SSDアルゴリズムとチャンク分割").
//
// Work-group: one batch row, one 256-token super-chunk (256/Q chunks) and KH
// heads of one B/C group; 4 waves. The super-chunk is cut into eight 32-row
// blocks l; wave w owns blocks w and 7-w so that the causal triangle splits
// evenly. For block l and every column block s <= l of the same chunk:
//   1. S^T = B_s C_l^T on MFMA (K = dstate; B and C rows are dstate-contiguous
//      in HBM, so both operands load straight from global memory; the C_l
//      fragments stay in registers for the whole block).
//   2. per head: multiply by exp(Acs_l - Acs_s) dt_s (factored per 32-block,
//      see below), mask s > l, round to bf16. The S^T tile comes out with
//      lane = column l and registers = rows s in runs of 4, which is exactly
//      the B operand of the next MFMA under a k permutation that the X^T
//      operand reproduces with two 8-byte LDS reads.
//   3. y^T += X^T G^T on MFMA, X^T (token-contiguous rows) staged in LDS once
//      per work-group through 8 x 8 register transposes.
// The output is produced transposed (rows p, lane = token l), so the
// state-entering term -- y^T = H_c^T C_l^T, computed first with H_c^T bf16
// straight from HBM -- takes its exp(Acs_l) factor as one multiplier per
// lane, and each lane stores 4 consecutive p at a time. The C B^T tile is
// computed once and used by the KH heads.
#include "mfma_util.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kSC = 256;          // tokens per super-chunk
constexpr int kXS = kSC + 4;      // X^T row stride (bf16): 520 B, 8-byte reads conflict-free
constexpr float kLog2e = 1.4426950408889634f;

template <int N, int P, int KH>
__global__ __launch_bounds__(kThreads) void chunk_scan_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const float* __restrict__ Acs, const float* __restrict__ dtq, const uint16_t* __restrict__ Hb,
    const float* __restrict__ D, uint16_t* __restrict__ y, int T, int H, int G, int Q, int nc,
    int nsc, int nhg) {
  __shared__ __attribute__((aligned(16))) uint16_t sXt[KH][P][kXS];
  __shared__ __attribute__((aligned(16))) float sA[KH][kSC];  // Acs * log2(e)
  __shared__ __attribute__((aligned(16))) float sF[KH][kSC];  // exp(Acs[block start] - Acs_s) * dt_s

  const int id = xcd_swizzle(blockIdx.x, gridDim.x);
  const int hg = id % nhg;
  const int bs = id / nhg;
  const int sc = bs % nsc, b = bs / nsc;
  const int h0 = hg * KH;
  const int g = h0 / (H / G);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int t0 = sc * kSC;
  const int c0 = sc * (kSC / Q);  // first chunk of the super-chunk
  const int lpc = Q / 32;         // 32-row blocks per chunk
  const bool full = t0 + kSC <= T;  // no token of this super-chunk is past the end

  // ---- stage Acs, the per-column decay factors and X^T of the KH heads.
  // Decay factorisation: for l, s in the same chunk, s in the 32-block that
  // starts at s0,  exp(Acs_l - Acs_s) = exp(Acs_l - Acs_s0) * exp(Acs_s0 - Acs_s);
  // the first factor is <= 1 (one exponential per lane and tile), the second
  // lies in [1, exp(32 * max |dt A|)] and is tabulated here with dt_s folded in.
  for (int e = tid; e < KH * kSC; e += kThreads) {
    const int kh = e / kSC, i = e % kSC;
    const int c = c0 + i / Q;
    float a = 0.f, f = 0.f;
    if (c < nc) {
      const size_t row = ((size_t(b) * H + h0 + kh) * nc + c) * Q;
      const int q = i % Q;
      a = Acs[row + q] * kLog2e;
      f = __builtin_amdgcn_exp2f(Acs[row + (q & ~31)] * kLog2e - a) * dtq[row + q];
    }
    sA[kh][i] = a;
    sF[kh][i] = f;
  }
  constexpr int NXB = (kSC / 8) * (P / 8);
  for (int blk = tid; blk < KH * NXB; blk += kThreads) {
    const int kh = blk / NXB, r = blk % NXB;
    const int tg = r / (P / 8), pg = r % (P / 8);
    u32x4 in[8], out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = min(t0 + 8 * tg + i, T - 1);
      in[i] = load16(x + ((size_t(b) * T + t) * H + h0 + kh) * P + 8 * pg);
    }
    if (!full) {
#pragma unroll
      for (int i = 0; i < 8; ++i) in[i] = keep_or_zero(t0 + 8 * tg + i < T, in[i]);
    }
    transpose8x8_b16(in, out);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x2* dst = reinterpret_cast<u32x2*>(&sXt[kh][8 * pg + j][8 * tg]);
      dst[0] = u32x2{out[j][0], out[j][1]};
      dst[1] = u32x2{out[j][2], out[j][3]};
    }
  }
  __syncthreads();

  for (int which = 0; which < 2; ++which) {
    const int i = which ? 7 - wave : wave;  // 32-row block of the super-chunk
    const int tl0 = t0 + 32 * i;
    if (tl0 >= T) continue;                 // wave-uniform: nothing to produce
    const int jfirst = (i / lpc) * lpc;     // first column block of the same chunk
    const int cg = c0 + i / lpc;            // global chunk index (< nc)
    const int lcol = 32 * i + l32;          // this lane's output row (token) in the super-chunk

    u32x4 cf[N / 16];                       // C rows of the block, k = dstate
    {
      const uint16_t* cr = Cm + ((size_t(b) * T + min(tl0 + l32, T - 1)) * G + g) * N + 8 * g2;
#pragma unroll
      for (int ks = 0; ks < N / 16; ++ks) cf[ks] = load16(cr + 16 * ks);
      if (!full) {
#pragma unroll
        for (int ks = 0; ks < N / 16; ++ks) cf[ks] = keep_or_zero(tl0 + l32 < T, cf[ks]);
      }
    }
    // B rows of column block j, k = dstate (row index clamped into the tensor;
    // rows past the end are zeroed where they are used, so the loads can stay
    // in flight). The next block's rows are loaded while the current one is
    // being used, unless that would cost occupancy (dstate 256: one batch per
    // iteration instead).
    auto load_b = [&](int j, u32x4 (&bf)[N / 16]) {
      const int ts = t0 + 32 * j + l32;
      const uint16_t* br = Bm + ((size_t(b) * T + min(ts, T - 1)) * G + g) * N + 8 * g2;
#pragma unroll
      for (int ks = 0; ks < N / 16; ++ks) bf[ks] = load16(br + 16 * ks);
    };
    constexpr bool kPrefetch = N <= 128;
    u32x4 bnext[N / 16];
    if (kPrefetch) load_b(jfirst, bnext);

    // ---- y^T = H_c^T C_l^T first (rows p, column l = this lane's token), then
    // scaled by exp(Acs_l): one multiplier per lane in this orientation
    f32x16 acc[KH][P / 32];
#pragma unroll
    for (int kh = 0; kh < KH; ++kh) {
      const uint16_t* hr = Hb + (((size_t(b) * nc + cg) * H + h0 + kh) * P + l32) * size_t(N) + 8 * g2;
#pragma unroll
      for (int pb = 0; pb < P / 32; ++pb) {
        f32x16 a = zero16();
#pragma unroll
        for (int ks = 0; ks < N / 16; ++ks)
          a = mfma32x32x16(load16(hr + size_t(32 * pb) * N + 16 * ks), cf[ks], a);
        acc[kh][pb] = a;
      }
      const float sl = __builtin_amdgcn_exp2f(sA[kh][lcol]);
#pragma unroll
      for (int pb = 0; pb < P / 32; ++pb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[kh][pb][r] *= sl;
    }

    // ---- y^T += X^T G^T over the column blocks of the chunk
    for (int j = jfirst; j <= i; ++j) {
      u32x4 bcur[N / 16];
      if (kPrefetch) {
#pragma unroll
        for (int ks = 0; ks < N / 16; ++ks) bcur[ks] = bnext[ks];
        if (j < i) load_b(j + 1, bnext);
      } else {
        load_b(j, bcur);
      }
      if (!full) {
        const bool jin = t0 + 32 * j + l32 < T;
#pragma unroll
        for (int ks = 0; ks < N / 16; ++ks) bcur[ks] = keep_or_zero(jin, bcur[ks]);
      }
      f32x16 sacc = zero16();
#pragma unroll
      for (int ks = 0; ks < N / 16; ++ks) sacc = mfma32x32x16(bcur[ks], cf[ks], sacc);  // rows s, column l
      const bool diag = (j == i);
#pragma unroll
      for (int kh = 0; kh < KH; ++kh) {
        // exp(Acs_l - Acs_{32j}) <= 1, once per lane and tile
        const float lfac = __builtin_amdgcn_exp2f(sA[kh][lcol] - sA[kh][32 * j]);
        uint32_t gw[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int sb = 32 * j + 8 * q + 4 * g2;  // rows sb .. sb+3 of register run q
          const f32x4 fs = *reinterpret_cast<const f32x4*>(&sF[kh][sb]);
          float v[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            float e = sacc[4 * q + rr] * lfac * fs[rr];
            if (diag && sb + rr > lcol) e = 0.f;   // causal mask (before any use of e)
            v[rr] = e;
          }
          gw[2 * q] = pack_bf16x2(v[0], v[1]);
          gw[2 * q + 1] = pack_bf16x2(v[2], v[3]);
        }
        const u32x4 ga = u32x4{gw[0], gw[1], gw[2], gw[3]};  // rows s = 32j + [0, 16)
        const u32x4 gb = u32x4{gw[4], gw[5], gw[6], gw[7]};  // rows s = 32j + [16, 32)
#pragma unroll
        for (int pb = 0; pb < P / 32; ++pb) {
          const uint16_t* xr = &sXt[kh][32 * pb + l32][32 * j + 4 * g2];
          const u32x2 x0 = *reinterpret_cast<const u32x2*>(xr);
          const u32x2 x1 = *reinterpret_cast<const u32x2*>(xr + 8);
          const u32x2 x2 = *reinterpret_cast<const u32x2*>(xr + 16);
          const u32x2 x3 = *reinterpret_cast<const u32x2*>(xr + 24);
          acc[kh][pb] = mfma32x32x16(u32x4{x0[0], x0[1], x1[0], x1[1]}, ga, acc[kh][pb]);
          acc[kh][pb] = mfma32x32x16(u32x4{x2[0], x2[1], x3[0], x3[1]}, gb, acc[kh][pb]);
        }
      }
    }

    // ---- epilogue: + D x, round, store 4 consecutive p (8 bytes) per run
    const int t = tl0 + l32;
    if (t < T) {
#pragma unroll
      for (int kh = 0; kh < KH; ++kh) {
        const float Dh = D ? D[h0 + kh] : 0.f;
        uint16_t* yr = y + ((size_t(b) * T + t) * H + h0 + kh) * P + 4 * g2;
#pragma unroll
        for (int pb = 0; pb < P / 32; ++pb) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int p = 32 * pb + 8 * q + 4 * g2;
            float o[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              o[rr] = acc[kh][pb][4 * q + rr] + Dh * bf16_to_f32(sXt[kh][p + rr][lcol]);
            *reinterpret_cast<u32x2*>(yr + 32 * pb + 8 * q) =
                u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          }
        }
      }
    }
  }
}

template <int N, int P, int KH>
hipError_t launch_t(const FwdShape& s, const void* x, const void* B, const void* C,
                    const float* Acs, const float* dtq, const uint16_t* Hb, const float* D, void* y,
                    hipStream_t st) {
  const int nsc = (s.T + kSC - 1) / kSC;
  const int nhg = s.H / KH;
  const long blocks = long(s.b) * nsc * nhg;
  hipLaunchKernelGGL((chunk_scan_mfma_kernel<N, P, KH>), dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(B),
                     static_cast<const uint16_t*>(C), Acs, dtq, Hb, D, static_cast<uint16_t*>(y), s.T,
                     s.H, s.G, s.Q, s.nc, nsc, nhg);
  return hipGetLastError();
}

template <int N, int P>
hipError_t launch_np(const FwdShape& s, const void* x, const void* B, const void* C,
                     const float* Acs, const float* dtq, const uint16_t* Hb, const float* D, void* y,
                     hipStream_t st) {
  // two heads share each C B^T tile while the X^T staging fits two work-groups per CU
  if constexpr (P <= 64) {
    if ((s.H / s.G) % 2 == 0) return launch_t<N, P, 2>(s, x, B, C, Acs, dtq, Hb, D, y, st);
  }
  return launch_t<N, P, 1>(s, x, B, C, Acs, dtq, Hb, D, y, st);
}

template <int N>
hipError_t launch_n(const FwdShape& s, const void* x, const void* B, const void* C,
                    const float* Acs, const float* dtq, const uint16_t* Hb, const float* D, void* y,
                    hipStream_t st) {
  switch (s.P) {
    case 32: return launch_np<N, 32>(s, x, B, C, Acs, dtq, Hb, D, y, st);
    case 64: return launch_np<N, 64>(s, x, B, C, Acs, dtq, Hb, D, y, st);
    case 128: return launch_np<N, 128>(s, x, B, C, Acs, dtq, Hb, D, y, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_scan_mfma(const FwdShape& s, const void* x, const void* B, const void* C,
                                  const float* Acs, const float* dtq, const uint16_t* Hb,
                                  const float* D, void* y, hipStream_t st) {
  switch (s.N) {
    case 32: return launch_n<32>(s, x, B, C, Acs, dtq, Hb, D, y, st);
    case 64: return launch_n<64>(s, x, B, C, Acs, dtq, Hb, D, y, st);
    case 128: return launch_n<128>(s, x, B, C, Acs, dtq, Hb, D, y, st);
    case 256: return launch_n<256>(s, x, B, C, Acs, dtq, Hb, D, y, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace ssd
