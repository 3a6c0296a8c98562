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
// Work-group: one batch row, one 256-token super-chunk (256/Q chunks), one
// head; 4 waves. The C B^T tiles come precomputed once per group
// (chunk_scores.hip) in MFMA-fragment order. The super-chunk is cut into eight
// 32-row blocks l; wave w owns blocks w and 7-w so that the causal triangle
// splits evenly. The output is produced transposed (y^T: rows p, lane = token
// l), which makes every per-token factor one multiplier per lane:
//   1. y^T = H_c^T C_l^T (k = dstate): H_c^T staged once in LDS (bf16, from
//      state_passing), C_l rows straight from HBM; then y^T *= exp(Acs_l).
//   2. for each column block s <= l of the chunk: the C B^T tile (lane =
//      column l, registers = rows s in runs of 4) times exp(Acs_l - Acs_s) dt_s
//      (factored per 32-block, see the staging below), masked to s <= l,
//      rounded to bf16, is the B operand of y^T += X^T G^T under a k
//      permutation that the X^T operand reproduces with two 8-byte LDS reads.
//      X^T (token-contiguous rows) is staged once per work-group through 8 x 8
//      register transposes.
//   3. + D x, bf16 rounding, 8-byte stores of 4 consecutive p.
#include "mfma_util.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kSC = 256;          // tokens per super-chunk
constexpr int kXS = kSC + 4;      // X^T row stride (bf16): 520 B, 8-byte reads conflict-free
constexpr float kLog2e = 1.4426950408889634f;

template <int N, int P>
__global__ __launch_bounds__(kThreads) void chunk_scan_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ CB, const uint16_t* __restrict__ Cm,
    const float* __restrict__ Acs, const float* __restrict__ dtq, const uint16_t* __restrict__ Hb,
    const float* __restrict__ D, uint16_t* __restrict__ y, int T, int H, int G, int Q, int nc,
    int nsc) {
  constexpr int kHS = N + 8;  // H^T row stride (bf16): 16-byte reads of 16 lanes hit distinct banks
  __shared__ __attribute__((aligned(16))) uint16_t sXt[P][kXS];
  __shared__ __attribute__((aligned(16))) uint16_t sHt[P][kHS];
  __shared__ __attribute__((aligned(16))) float sA[kSC];  // Acs * log2(e)
  __shared__ __attribute__((aligned(16))) float sF[kSC];  // exp(Acs[block start] - Acs_s) * dt_s

  const int id = xcd_swizzle(blockIdx.x, gridDim.x);
  const int h = id % H;
  const int bs = id / H;
  const int sc = bs % nsc, b = bs / nsc;
  const int g = h / (H / G);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int t0 = sc * kSC;
  const int cps = kSC / Q;        // chunks per super-chunk
  const int c0 = sc * cps;        // first chunk of the super-chunk
  const int lpc = Q / 32;         // 32-row blocks per chunk
  const int ntile = lpc * (lpc + 1) / 2;
  const bool full = t0 + kSC <= T;     // no token of this super-chunk is past the end
  const bool hlds = cps == 1;          // one chunk: its H_c^T fits in LDS

  // ---- staging. Decay factorisation: for l, s in the same chunk, s in the
  // 32-block that starts at s0,  exp(Acs_l - Acs_s) = exp(Acs_l - Acs_s0) * exp(Acs_s0 - Acs_s);
  // the first factor is <= 1 (one exponential per lane and tile), the second
  // lies in [1, exp(32 * max |dt A|)] and is tabulated here with dt_s folded in.
  for (int i = tid; i < kSC; i += kThreads) {
    const int c = c0 + i / Q;
    float a = 0.f, f = 0.f;
    if (c < nc) {
      const size_t row = ((size_t(b) * H + h) * nc + c) * Q;
      const int q = i % Q;
      a = Acs[row + q] * kLog2e;
      f = __builtin_amdgcn_exp2f(Acs[row + (q & ~31)] * kLog2e - a) * dtq[row + q];
    }
    sA[i] = a;
    sF[i] = f;
  }
  if (hlds) {
    const uint16_t* hsrc = Hb + ((size_t(b) * nc + c0) * H + h) * size_t(P) * N;
    for (int e = tid; e < P * (N / 8); e += kThreads) {
      const int p = e / (N / 8), seg = e % (N / 8);
      *reinterpret_cast<u32x4*>(&sHt[p][8 * seg]) = load16(hsrc + size_t(p) * N + 8 * seg);
    }
  }
  constexpr int NXB = (kSC / 8) * (P / 8);
  for (int blk = tid; blk < NXB; blk += kThreads) {
    const int tg = blk / (P / 8), pg = blk % (P / 8);
    u32x4 in[8], out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = min(t0 + 8 * tg + i, T - 1);
      in[i] = load16(x + ((size_t(b) * T + t) * H + h) * P + 8 * pg);
    }
    if (!full) {
#pragma unroll
      for (int i = 0; i < 8; ++i) in[i] = keep_or_zero(t0 + 8 * tg + i < T, in[i]);
    }
    transpose8x8_b16(in, out);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u32x2* dst = reinterpret_cast<u32x2*>(&sXt[8 * pg + j][8 * tg]);
      dst[0] = u32x2{out[j][0], out[j][1]};
      dst[1] = u32x2{out[j][2], out[j][3]};
    }
  }
  __syncthreads();

  const float Dh = D ? D[h] : 0.f;
  for (int which = 0; which < 2; ++which) {
    const int i = which ? 7 - wave : wave;  // 32-row block of the super-chunk
    const int tl0 = t0 + 32 * i;
    if (tl0 >= T) continue;                 // wave-uniform: nothing to produce
    const int jfirst = (i / lpc) * lpc;     // first column block of the same chunk
    const int cg = c0 + i / lpc;            // global chunk index (< nc)
    const int lcol = 32 * i + l32;          // this lane's output token in the super-chunk
    const int irel = i - jfirst;
    const uint16_t* tiles = CB + (((size_t(b) * nc + cg) * G + g) * ntile + size_t(irel) * (irel + 1) / 2) * 1024 +
                            size_t(lane) * 16;
    auto load_tile = [&](int j, u32x4 (&t)[2]) {
      const u32x4* src = reinterpret_cast<const u32x4*>(tiles + size_t(j - jfirst) * 1024);
      t[0] = src[0];
      t[1] = src[1];
    };
    u32x4 tnext[2];
    load_tile(jfirst, tnext);

    // ---- y^T = H_c^T C_l^T, then * exp(Acs_l)
    u32x4 cf[N / 16];
    {
      const uint16_t* cr = Cm + ((size_t(b) * T + min(tl0 + l32, T - 1)) * G + g) * N + 8 * g2;
#pragma unroll
      for (int ks = 0; ks < N / 16; ++ks) cf[ks] = load16(cr + 16 * ks);
      if (!full) {
#pragma unroll
        for (int ks = 0; ks < N / 16; ++ks) cf[ks] = keep_or_zero(tl0 + l32 < T, cf[ks]);
      }
    }
    f32x16 acc[P / 32];
    const uint16_t* hg = Hb + (((size_t(b) * nc + cg) * H + h) * P + l32) * size_t(N) + 8 * g2;
#pragma unroll
    for (int pb = 0; pb < P / 32; ++pb) {
      f32x16 a = zero16();
#pragma unroll
      for (int ks = 0; ks < N / 16; ++ks) {
        const u32x4 hf = hlds ? *reinterpret_cast<const u32x4*>(&sHt[32 * pb + l32][16 * ks + 8 * g2])
                              : load16(hg + size_t(32 * pb) * N + 16 * ks);
        a = mfma32x32x16(hf, cf[ks], a);
      }
      const float sl = __builtin_amdgcn_exp2f(sA[lcol]);
#pragma unroll
      for (int r = 0; r < 16; ++r) a[r] *= sl;
      acc[pb] = a;
    }

    // ---- y^T += X^T G^T over the column blocks of the chunk
    for (int j = jfirst; j <= i; ++j) {
      u32x4 tcur[2] = {tnext[0], tnext[1]};
      if (j < i) load_tile(j + 1, tnext);
      const bool diag = (j == i);
      // exp(Acs_l - Acs_{32j}) <= 1, once per lane and tile
      const float lfac = __builtin_amdgcn_exp2f(sA[lcol] - sA[32 * j]);
      uint32_t gw[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int sb = 32 * j + 8 * q + 4 * g2;  // rows sb .. sb+3 of register run q
        const f32x4 fs = *reinterpret_cast<const f32x4*>(&sF[sb]);
        const uint32_t w0 = tcur[q / 2][2 * (q % 2)], w1 = tcur[q / 2][2 * (q % 2) + 1];
        const float cb[4] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1)};
        float v[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          float e = cb[rr] * lfac * fs[rr];
          if (diag && sb + rr > lcol) e = 0.f;   // causal mask
          v[rr] = e;
        }
        gw[2 * q] = pack_bf16x2(v[0], v[1]);
        gw[2 * q + 1] = pack_bf16x2(v[2], v[3]);
      }
      const u32x4 ga = u32x4{gw[0], gw[1], gw[2], gw[3]};  // rows s = 32j + [0, 16)
      const u32x4 gb = u32x4{gw[4], gw[5], gw[6], gw[7]};  // rows s = 32j + [16, 32)
#pragma unroll
      for (int pb = 0; pb < P / 32; ++pb) {
        const uint16_t* xr = &sXt[32 * pb + l32][32 * j + 4 * g2];
        const u32x2 x0 = *reinterpret_cast<const u32x2*>(xr);
        const u32x2 x1 = *reinterpret_cast<const u32x2*>(xr + 8);
        const u32x2 x2 = *reinterpret_cast<const u32x2*>(xr + 16);
        const u32x2 x3 = *reinterpret_cast<const u32x2*>(xr + 24);
        acc[pb] = mfma32x32x16(u32x4{x0[0], x0[1], x1[0], x1[1]}, ga, acc[pb]);
        acc[pb] = mfma32x32x16(u32x4{x2[0], x2[1], x3[0], x3[1]}, gb, acc[pb]);
      }
    }

    // ---- epilogue: + D x, round, store 4 consecutive p (8 bytes) per run
    const int t = tl0 + l32;
    if (t < T) {
      uint16_t* yr = y + ((size_t(b) * T + t) * H + h) * P + 4 * g2;
#pragma unroll
      for (int pb = 0; pb < P / 32; ++pb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int p = 32 * pb + 8 * q + 4 * g2;
          float o[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            o[rr] = acc[pb][4 * q + rr] + Dh * bf16_to_f32(sXt[p + rr][lcol]);
          *reinterpret_cast<u32x2*>(yr + 32 * pb + 8 * q) =
              u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        }
      }
    }
  }
}

template <int N, int P>
hipError_t launch_np(const FwdShape& s, const void* x, const uint16_t* CB, const void* C,
                     const float* Acs, const float* dtq, const uint16_t* Hb, const float* D, void* y,
                     hipStream_t st) {
  const int nsc = (s.T + kSC - 1) / kSC;
  const long blocks = long(s.b) * nsc * s.H;
  hipLaunchKernelGGL((chunk_scan_mfma_kernel<N, P>), dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                     static_cast<const uint16_t*>(x), CB, static_cast<const uint16_t*>(C), Acs, dtq, Hb,
                     D, static_cast<uint16_t*>(y), s.T, s.H, s.G, s.Q, s.nc, nsc);
  return hipGetLastError();
}

template <int N>
hipError_t launch_n(const FwdShape& s, const void* x, const uint16_t* CB, const void* C,
                    const float* Acs, const float* dtq, const uint16_t* Hb, const float* D, void* y,
                    hipStream_t st) {
  switch (s.P) {
    case 32: return launch_np<N, 32>(s, x, CB, C, Acs, dtq, Hb, D, y, st);
    case 64: return launch_np<N, 64>(s, x, CB, C, Acs, dtq, Hb, D, y, st);
    case 128: return launch_np<N, 128>(s, x, CB, C, Acs, dtq, Hb, D, y, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_scan_mfma(const FwdShape& s, const void* x, const uint16_t* CB,
                                  const void* C, const float* Acs, const float* dtq,
                                  const uint16_t* Hb, const float* D, void* y, hipStream_t st) {
  switch (s.N) {
    case 32: return launch_n<32>(s, x, CB, C, Acs, dtq, Hb, D, y, st);
    case 64: return launch_n<64>(s, x, CB, C, Acs, dtq, Hb, D, y, st);
    case 128: return launch_n<128>(s, x, CB, C, Acs, dtq, Hb, D, y, st);
    case 256: return launch_n<256>(s, x, CB, C, Acs, dtq, Hb, D, y, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace ssd
