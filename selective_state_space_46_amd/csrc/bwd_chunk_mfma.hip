// bwd_chunk_mfma.hip -- the per-chunk gradients of the chunked forward, on the
// bf16 matrix cores.
//
// Inside one chunk (tokens s <= l, decays e_ls = exp(Acs_l - Acs_s), chunk
// end Q-1, H_c the state entering the chunk, G_c the gradient of the state
// leaving it) the forward is (youngju.dev "Mamba / selective SSM",
// "SSDアルゴリズムとチャンク分割"; the chunk product of "State Space Dualityの発見")
//   y_l  = sum_{s<=l} (C_l . B_s) e_ls dt_s x_s + exp(Acs_l) C_l^T H_c + D x_l
//   H_{c+1} = exp(Acs_{Q-1}) H_c + sum_s e_{Q-1,s} dt_s B_s x_s^T
// and its gradients for one head, with Sxy_sl = x_s . dy_l, are
//   dx_s  = sum_{l>=s} (C_l . B_s) e_ls dt_s dy_l + dt_s e_{Q-1,s} G_c^T B_s + D dy_s
//   dB'_s = sum_{l>=s} e_ls Sxy_sl C_l + e_{Q-1,s} G_c x_s          (dB_s = dt_s dB'_s)
//   dC_l  = sum_{s<=l} e_ls dt_s Sxy_sl B_s + exp(Acs_l) H_c dy_l
// The decay exponents get (the row and column sums of the quadratic form)
//   dAcs_t = C_t . dC_t - dt_t (B_t . dB'_t) + [t = Q-1] <G_c, H_{c+1}>
// where, with H_{c+1} = exp(Acs_{Q-1}) H_c + sum_s e_{Q-1,s} dt_s B_s x_s^T,
//   <G_c, H_{c+1}> = exp(Acs_{Q-1}) <G_c, H_c> + sum_s dt_s B_s . (e_{Q-1,s} G_c x_s)
// is formed from the same per-token state dots that the second term
// subtracts, so those cancel exactly in the reverse sum.
// whose in-chunk parts are the row and column sums of W_ls = (C_l . B_s) e_ls
// Sxy_sl (dt_s W_ls summed over s for C_l . dC_l, W_ls over l for B_s . dB'_s).
// In the reverse cumulative sum below most of those cancel (the diagonal
// exactly), so both are taken in fp32 from the same fp32 products (fp32 C B^T
// tiles from the recomputation), never from the bf16 operands of the dB' / dC
// contractions; likewise H_c enters the state term of dC as a bf16 pair
// hi + lo, so that C_l . dC_l keeps fp32 accuracy.
// and, since Acs_t = A sum_{k<=t} dt_k,
//   ddt_t = B_t . dB'_t + A R_t,  dA = sum_t dt_t R_t,  R_t = sum_{t'>=t} dAcs_t'.
// dB and dC of one head go out as fp32 partials; a later kernel sums the
// heads of each group (and dA, dD over the chunks) in a fixed order.
//
// Work-group: one (batch, chunk, head), 2 NB waves for NB 32-token blocks
// (Q = 32 NB). Wave i < NB owns block i as the s side (dx, dB': tiles of
// l-blocks j >= i); wave NB + i owns it as the l side (dC: tiles of s-blocks
// j <= i); every wave sees NB + 1 tiles' worth of work. The s side works in
// tiles whose lanes are tokens s (registers over rows l), so its two
// contractions over l take the tile as the B operand under the k permutation
// the A operand reproduces with transposed LDS reads (as chunk_scan does);
// the l side mirrors it with lanes = l. C B^T comes from the recomputation,
// already in the s-lane orientation. Every decay factor has a non-positive
// exponent (off the diagonal split at a block boundary, on it masked).
#include <type_traits>

#include "mfma_util.h"

namespace ssd {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int N, int P, int NB>
__global__ __launch_bounds__(128 * NB) void bwd_chunk_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const uint16_t* __restrict__ dy, const float* __restrict__ Acs, const float* __restrict__ dtq,
    const float* __restrict__ CBf, const float* __restrict__ CBt, const float* __restrict__ Hst,
    const uint16_t* __restrict__ Gb, const uint16_t* __restrict__ GbT,
    const float* __restrict__ ghp, const float* __restrict__ A, const float* __restrict__ D,
    uint16_t* __restrict__ dx, uint16_t* __restrict__ ddt, float* __restrict__ dBp, float* __restrict__ dCp,
    float* __restrict__ dAp, float* __restrict__ dDp, int T, int H, int G, int nc, int nghp) {
  constexpr int Q = 32 * NB;
  constexpr int kThr = 128 * NB;
  constexpr int RBP = P / 8, RBN = N / 8;   // 16-byte chunks per row
  constexpr int ntile = NB * (NB + 1) / 2;
  __shared__ __attribute__((aligned(16))) uint16_t sDY[Q * P];
  __shared__ __attribute__((aligned(16))) uint16_t sB[Q * N];
  __shared__ __attribute__((aligned(16))) uint16_t sC[Q * N];
  __shared__ __attribute__((aligned(16))) uint16_t sH[P * N];
  __shared__ __attribute__((aligned(16))) uint16_t sHlo[P * N];   // H_c - bf16(H_c), rounded
  __shared__ float sA2[Q], sdt[Q], sF[Q], sL[Q], sEL[Q], sEl[Q];
  __shared__ float sds[Q], sdl[Q], sdd[Q], sdst[Q];
  __shared__ float sred[2 * NB][2];

  const int id = xcd_swizzle(blockIdx.x, gridDim.x);
  const int h = id % H;
  const int bc = id / H;
  const int c = bc % nc, b = bc / nc;
  const int g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_id();
  const int l32 = lane & 31, g2 = lane >> 5;
  const long r0 = long(b) * T + long(c) * Q;        // first token row of the chunk
  const int nv = min(Q, T - c * Q);                 // valid tokens
  const size_t arow = ((size_t(b) * H + h) * nc + c) * Q;
  const size_t sbase = ((size_t(b) * nc + c) * H + h) * size_t(P) * N;

  // ---- tables (exponents in base 2)
  for (int t = tid; t < Q; t += kThr) {
    const float a2 = Acs[arow + t] * kLog2e, d = dtq[arow + t];
    sA2[t] = a2;
    sdt[t] = d;
    sF[t] = __builtin_amdgcn_exp2f(Acs[arow + (t | 31)] * kLog2e - a2) * d;   // <= dt
    sL[t] = __builtin_amdgcn_logf(d) - a2;                                     // -inf where dt = 0
    sEL[t] = __builtin_amdgcn_exp2f(a2 - Acs[arow + (t & ~31)] * kLog2e);    // <= 1
    sEl[t] = __builtin_amdgcn_exp2f(Acs[arow + Q - 1] * kLog2e - a2);         // <= 1
  }
  // ---- natural row-major tiles: dy, B, C (rows past the chunk are zeros), H_c (hi and lo)
  for (int e = tid; e < Q * RBP; e += kThr) {
    const int r = e / RBP, cc = e % RBP;
    const u32x4 v = load16(dy + ((r0 + min(r, nv - 1)) * H + h) * size_t(P) + 8 * cc);
    *reinterpret_cast<u32x4*>(&sDY[lds_off<RBP>(r, 8 * cc)]) = keep_or_zero(r < nv, v);
  }
  for (int e = tid; e < Q * RBN; e += kThr) {
    const int r = e / RBN, cc = e % RBN;
    const size_t ro = ((r0 + min(r, nv - 1)) * G + g) * size_t(N) + 8 * cc;
    *reinterpret_cast<u32x4*>(&sB[lds_off<RBN>(r, 8 * cc)]) = keep_or_zero(r < nv, load16(Bm + ro));
    *reinterpret_cast<u32x4*>(&sC[lds_off<RBN>(r, 8 * cc)]) = keep_or_zero(r < nv, load16(Cm + ro));
  }
  for (int e = tid; e < P * RBN; e += kThr) {
    const int r = e / RBN, cc = e % RBN;
    const f32x4 h0 = *reinterpret_cast<const f32x4*>(Hst + sbase + size_t(r) * N + 8 * cc);
    const f32x4 h1 = *reinterpret_cast<const f32x4*>(Hst + sbase + size_t(r) * N + 8 * cc + 4);
    const u32x4 hi = u32x4{pack_bf16x2(h0[0], h0[1]), pack_bf16x2(h0[2], h0[3]), pack_bf16x2(h1[0], h1[1]),
                           pack_bf16x2(h1[2], h1[3])};
    const u32x4 lo = u32x4{pack_bf16x2(h0[0] - bf16_lo(hi[0]), h0[1] - bf16_hi(hi[0])),
                           pack_bf16x2(h0[2] - bf16_lo(hi[1]), h0[3] - bf16_hi(hi[1])),
                           pack_bf16x2(h1[0] - bf16_lo(hi[2]), h1[1] - bf16_hi(hi[2])),
                           pack_bf16x2(h1[2] - bf16_lo(hi[3]), h1[3] - bf16_hi(hi[3]))};
    *reinterpret_cast<u32x4*>(&sH[lds_off<RBN>(r, 8 * cc)]) = hi;
    *reinterpret_cast<u32x4*>(&sHlo[lds_off<RBN>(r, 8 * cc)]) = lo;
  }
  __syncthreads();

  // lane constants of the permuted transposed reads (k = rows of a 32-row
  // block, in the order of the accumulator rows), per 32-column block
  const int q16 = lane & 15;
  const int mcol = 16 * ((lane >> 4) & 1) + 4 * (q16 & 3);
  auto toff = [&](auto rb, int u, int mt) {
    constexpr int RB = decltype(rb)::value;
    return lds_off<RB>(4 * g2 + 8 * u + (q16 >> 2), 32 * mt + mcol);
  };
  using RBPc = std::integral_constant<int, RBP>;
  using RBNc = std::integral_constant<int, RBN>;

  const float Ah = A[h];
  const float Dh = D ? D[h] : 0.f;

  if (wave < NB) {
    // ================= s side: block i as the tokens s
    const int i = wave;
    const int s = 32 * i + l32;
    const bool sok = s < nv;
    const long srow = r0 + min(s, nv - 1);
    const float dts = sdt[s], a2s = sA2[s], els = sEl[s];
    u32x4 xr[P / 16];
#pragma unroll
    for (int kk = 0; kk < P / 16; ++kk)
      xr[kk] = keep_or_zero(sok, load16(x + (srow * H + h) * size_t(P) + 16 * kk + 8 * g2));

    f32x16 adx[P / 32], adb[N / 32];
    // state terms: dx^T(p, s) = sum_n G(n, p) B_s[n];  dB'^T(n, s) = sum_p G(n, p) x_s[p]
#pragma unroll
    for (int pt = 0; pt < P / 32; ++pt) {
      adx[pt] = zero16();
#pragma unroll
      for (int kk = 0; kk < N / 16; ++kk) {
        const u32x4 ga = load16(Gb + sbase + size_t(32 * pt + l32) * N + 16 * kk + 8 * g2);
        const u32x4 bs = keep_or_zero(sok, load16(Bm + (srow * G + g) * size_t(N) + 16 * kk + 8 * g2));
        adx[pt] = mfma32x32x16(ga, bs, adx[pt]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) adx[pt][r] *= dts * els;
    }
#pragma unroll
    for (int nt = 0; nt < N / 32; ++nt) {
      adb[nt] = zero16();
#pragma unroll
      for (int kk = 0; kk < P / 16; ++kk) {
        const u32x4 ga = load16(GbT + sbase + size_t(32 * nt + l32) * P + 16 * kk + 8 * g2);   // G rows n
        adb[nt] = mfma32x32x16(ga, xr[kk], adb[nt]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) adb[nt][r] *= els;
    }
    // B_s . dB'_s of the state term (rows n = 32 nt + 8 q + 4 g2 + 0..3 of lane s)
    float bd = 0.f;
#pragma unroll
    for (int nt = 0; nt < N / 32; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = 32 * nt + 8 * q + 4 * g2;
        const u32x2 bv = *reinterpret_cast<const u32x2*>(Bm + (srow * G + g) * size_t(N) + n);
        bd += adb[nt][4 * q] * bf16_lo(bv[0]) + adb[nt][4 * q + 1] * bf16_hi(bv[0]) +
              adb[nt][4 * q + 2] * bf16_lo(bv[1]) + adb[nt][4 * q + 3] * bf16_hi(bv[1]);
      }
    const float bdst = bd + __shfl_xor(bd, 32, 64);   // the state term's B_s . dB'_s

    // intra-chunk terms, one 32 x 32 tile (rows l of block j, lanes s) at a time;
    // l-blocks wholly past the valid tokens add nothing (dy = 0 there) and
    // their C B^T tiles are never computed
    const int jend = min(NB, (nv + 31) / 32);
    for (int j = i; j < jend; ++j) {
      const int lrow_l = 32 * j + l32;
      f32x16 accS = zero16();
#pragma unroll
      for (int kk = 0; kk < P / 16; ++kk) {
        const u32x4 dyl = keep_or_zero(lrow_l < nv, load16(dy + ((r0 + min(lrow_l, nv - 1)) * H + h) * size_t(P) +
                                                         16 * kk + 8 * g2));
        accS = mfma32x32x16(dyl, xr[kk], accS);                         // Sxy^T: rows l, lane s
      }
      const f32x4* tsrc = reinterpret_cast<const f32x4*>(
          CBt + (((size_t(b) * nc + c) * G + g) * ntile + size_t(j) * (j + 1) / 2 + i) * 1024 + size_t(lane) * 16);
      const f32x4 cb4[4] = {tsrc[0], tsrc[1], tsrc[2], tsrc[3]};   // C_l . B_s, rows l in accumulator order
      const bool diag = j == i;
      const float lf = diag ? 0.f : __builtin_amdgcn_exp2f(sA2[32 * j] - a2s);
      uint32_t zw[8], mw[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float cb_lo = cb4[m / 2][2 * (m % 2)], cb_hi = cb4[m / 2][2 * (m % 2) + 1];
        float e2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = 2 * m + u;
          const int l = 32 * j + 8 * (r / 4) + 4 * g2 + (r % 4);
          if (diag) {
            const float ex = __builtin_amdgcn_exp2f(fminf(sA2[l] - a2s, 0.f));
            e2[u] = l >= s ? ex : 0.f;
          } else {
            e2[u] = sEL[l] * lf;
          }
        }
        const float z0 = e2[0] * accS[2 * m], z1 = e2[1] * accS[2 * m + 1];
        bd += z0 * cb_lo + z1 * cb_hi;                              // column sum of W
        zw[m] = pack_bf16x2(z0, z1);
        mw[m] = pack_bf16x2(e2[0] * dts * cb_lo, e2[1] * dts * cb_hi);
      }
      const u32x4 zga = u32x4{zw[0], zw[1], zw[2], zw[3]}, zgb = u32x4{zw[4], zw[5], zw[6], zw[7]};
      const u32x4 mga = u32x4{mw[0], mw[1], mw[2], mw[3]}, mgb = u32x4{mw[4], mw[5], mw[6], mw[7]};
      // dx^T(p, s) += sum_l dy^T(p, l) M(l, s)
      const int joP = 32 * j * P;
#pragma unroll
      for (int pt = 0; pt < P / 32; ++pt) {
        const int o0 = toff(RBPc{}, 0, pt) + joP, o1 = toff(RBPc{}, 1, pt) + joP;
        const u32x2 a0 = lds_read_tr16(sDY, o0), a1 = lds_read_tr16(sDY, o1);
        const u32x2 b0 = lds_read_tr16(sDY, o0 + 16 * P), b1 = lds_read_tr16(sDY, o1 + 16 * P);
        adx[pt] = mfma32x32x16(u32x4{a0[0], a0[1], a1[0], a1[1]}, mga, adx[pt]);
        adx[pt] = mfma32x32x16(u32x4{b0[0], b0[1], b1[0], b1[1]}, mgb, adx[pt]);
      }
      // dB'^T(n, s) += sum_l C^T(n, l) Z(l, s)
      const int joN = 32 * j * N;
#pragma unroll
      for (int nt = 0; nt < N / 32; ++nt) {
        const int o0 = toff(RBNc{}, 0, nt) + joN, o1 = toff(RBNc{}, 1, nt) + joN;
        const u32x2 a0 = lds_read_tr16(sC, o0), a1 = lds_read_tr16(sC, o1);
        const u32x2 b0 = lds_read_tr16(sC, o0 + 16 * N), b1 = lds_read_tr16(sC, o1 + 16 * N);
        adb[nt] = mfma32x32x16(u32x4{a0[0], a0[1], a1[0], a1[1]}, zga, adb[nt]);
        adb[nt] = mfma32x32x16(u32x4{b0[0], b0[1], b1[0], b1[1]}, zgb, adb[nt]);
      }
    }

    // dx = ... + D dy (rows p = 32 pt + 8 q + 4 g2 + 0..3 of lane s), stored as bf16
#pragma unroll
    for (int pt = 0; pt < P / 32; ++pt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int p = 32 * pt + 8 * q + 4 * g2;
        const u32x2 dv = *reinterpret_cast<const u32x2*>(dy + (srow * H + h) * size_t(P) + p);
        const float v0 = adx[pt][4 * q] + Dh * bf16_lo(dv[0]), v1 = adx[pt][4 * q + 1] + Dh * bf16_hi(dv[0]);
        const float v2 = adx[pt][4 * q + 2] + Dh * bf16_lo(dv[1]), v3 = adx[pt][4 * q + 3] + Dh * bf16_hi(dv[1]);
        if (sok)
          *reinterpret_cast<u32x2*>(dx + (srow * H + h) * size_t(P) + p) =
              u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
      }
    // dB_s = dt_s dB'_s as an fp32 partial of this head
#pragma unroll
    for (int nt = 0; nt < N / 32; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = 32 * nt + 8 * q + 4 * g2;
        if (sok)
          *reinterpret_cast<f32x4*>(dBp + (srow * H + h) * size_t(N) + n) =
              f32x4{dts * adb[nt][4 * q], dts * adb[nt][4 * q + 1], dts * adb[nt][4 * q + 2],
                    dts * adb[nt][4 * q + 3]};
      }
    bd += __shfl_xor(bd, 32, 64);
    // dy_s . x_s (for dD)
    float dd = 0.f;
#pragma unroll
    for (int kk = 0; kk < P / 16; ++kk) {
      const u32x4 dv = keep_or_zero(sok, load16(dy + (srow * H + h) * size_t(P) + 16 * kk + 8 * g2));
#pragma unroll
      for (int w = 0; w < 4; ++w)
        dd += bf16_lo(dv[w]) * bf16_lo(xr[kk][w]) + bf16_hi(dv[w]) * bf16_hi(xr[kk][w]);
    }
    dd += __shfl_xor(dd, 32, 64);
    if (g2 == 0) {
      sds[s] = sok ? bd : 0.f;
      sdst[s] = sok ? dts * bdst : 0.f;
      sdd[s] = dd;
    }
  } else {
    // ================= l side: block i as the tokens l
    const int i = wave - NB;
    const int l = 32 * i + l32;
    const bool lok = l < nv;
    const long lrow = r0 + min(l, nv - 1);
    const float a2l = sA2[l];
    u32x4 dyr[P / 16];
#pragma unroll
    for (int kk = 0; kk < P / 16; ++kk)
      dyr[kk] = keep_or_zero(lok, load16(dy + (lrow * H + h) * size_t(P) + 16 * kk + 8 * g2));
    // state term: dC^T(n, l) = exp(Acs_l) sum_p H(n, p) dy_l[p]
    f32x16 adc[N / 32];
    const float el = __builtin_amdgcn_exp2f(a2l);
#pragma unroll
    for (int nt = 0; nt < N / 32; ++nt) {
      adc[nt] = zero16();
#pragma unroll
      for (int kk = 0; kk < P / 16; ++kk) {
        const int kb = 16 * kk + 8 * g2;
        adc[nt] = mfma32x32x16(frag_tr<RBN>(sH, kb, kb + 4, 32 * nt, lane), dyr[kk], adc[nt]);
        adc[nt] = mfma32x32x16(frag_tr<RBN>(sHlo, kb, kb + 4, 32 * nt, lane), dyr[kk], adc[nt]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) adc[nt][r] *= el;
    }
    // C_l . dC_l of the state term
    float cd = 0.f;
#pragma unroll
    for (int nt = 0; nt < N / 32; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = 32 * nt + 8 * q + 4 * g2;
        const u32x2 cv = *reinterpret_cast<const u32x2*>(Cm + (lrow * G + g) * size_t(N) + n);
        cd += adc[nt][4 * q] * bf16_lo(cv[0]) + adc[nt][4 * q + 1] * bf16_hi(cv[0]) +
              adc[nt][4 * q + 2] * bf16_lo(cv[1]) + adc[nt][4 * q + 3] * bf16_hi(cv[1]);
      }
    // intra-chunk terms, tiles of rows s (block j) and lanes l (none when the
    // whole block l is past the valid tokens)
    const int jlast = 32 * i < nv ? i : -1;
    for (int j = 0; j <= jlast; ++j) {
      const int srw = 32 * j + l32;
      f32x16 accS = zero16();
#pragma unroll
      for (int kk = 0; kk < P / 16; ++kk) {
        const u32x4 xs = keep_or_zero(srw < nv, load16(x + ((r0 + min(srw, nv - 1)) * H + h) * size_t(P) +
                                                       16 * kk + 8 * g2));
        accS = mfma32x32x16(xs, dyr[kk], accS);                         // Sxy: rows s, lane l
      }
      const bool diag = j == i;
      const float lfac = diag ? 0.f : __builtin_amdgcn_exp2f(a2l - sA2[32 * j + 31]);
      // C B^T in the forward orientation (rows s, lane l)
      const f32x4* fsrc = reinterpret_cast<const f32x4*>(
          CBf + (((size_t(b) * nc + c) * G + g) * ntile + size_t(i) * (i + 1) / 2 + j) * 1024 + size_t(lane) * 16);
      const f32x4 cf4[4] = {fsrc[0], fsrc[1], fsrc[2], fsrc[3]};
      uint32_t zw[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float cf_lo = cf4[m / 2][2 * (m % 2)], cf_hi = cf4[m / 2][2 * (m % 2) + 1];
        float z2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = 2 * m + u;
          const int sr = 32 * j + 8 * (r / 4) + 4 * g2 + (r % 4);
          float dec;
          if (diag) {
            const float pv = __builtin_amdgcn_exp2f(a2l + sL[sr]);   // exp(Acs_l - Acs_s) dt_s
            dec = sr <= l ? pv : 0.f;
          } else {
            dec = lfac * sF[sr];
          }
          z2[u] = dec * accS[r];
        }
        cd += z2[0] * cf_lo + z2[1] * cf_hi;                          // row sum of dt W
        zw[m] = pack_bf16x2(z2[0], z2[1]);
      }
      const u32x4 zga = u32x4{zw[0], zw[1], zw[2], zw[3]}, zgb = u32x4{zw[4], zw[5], zw[6], zw[7]};
      const int joN = 32 * j * N;
#pragma unroll
      for (int nt = 0; nt < N / 32; ++nt) {
        const int o0 = toff(RBNc{}, 0, nt) + joN, o1 = toff(RBNc{}, 1, nt) + joN;
        const u32x2 a0 = lds_read_tr16(sB, o0), a1 = lds_read_tr16(sB, o1);
        const u32x2 b0 = lds_read_tr16(sB, o0 + 16 * N), b1 = lds_read_tr16(sB, o1 + 16 * N);
        adc[nt] = mfma32x32x16(u32x4{a0[0], a0[1], a1[0], a1[1]}, zga, adc[nt]);
        adc[nt] = mfma32x32x16(u32x4{b0[0], b0[1], b1[0], b1[1]}, zgb, adc[nt]);
      }
    }
    // dC_l as an fp32 partial of this head
#pragma unroll
    for (int nt = 0; nt < N / 32; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = 32 * nt + 8 * q + 4 * g2;
        if (lok)
          *reinterpret_cast<f32x4*>(dCp + (lrow * H + h) * size_t(N) + n) =
              f32x4{adc[nt][4 * q], adc[nt][4 * q + 1], adc[nt][4 * q + 2], adc[nt][4 * q + 3]};
      }
    cd += __shfl_xor(cd, 32, 64);
    if (g2 == 0) sdl[l] = lok ? cd : 0.f;
  }
  __syncthreads();

  // ---- dAcs, its reverse cumulative sum R, ddt, and this chunk's dA / dD
  //      terms: thread k < Q takes token t = Q-1-k, so an inclusive scan over k
  //      is the sum over t' >= t. The chunk-end term (dAcs_{Q-1} only, so a
  //      constant K added to every R_t) is a block sum: the per-token state
  //      dots and exp(Acs_{Q-1}) <G_c, H_c> from the reverse pass's partials.
  float dacs = 0.f, dtv = 0.f, ddv = 0.f, sdsv = 0.f, kpart = 0.f;
  const int t = Q - 1 - tid;
  if (tid < Q) {
    dtv = sdt[t];
    sdsv = sds[t];
    ddv = sdd[t];
    dacs = sdl[t] - dtv * sdsv;
    kpart = sdst[t];
  }
  if (tid < nghp)
    kpart += __builtin_amdgcn_exp2f(sA2[Q - 1]) * ghp[((size_t(b) * H + h) * nc + c) * nghp + tid];
  float v = dacs;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) kpart += __shfl_xor(kpart, off, 64);
  if (lane == 63) sred[wave][0] = v;
  if (lane == 0) sred[wave][1] = kpart;
  __syncthreads();
  float K = 0.f;
  for (int w = 0; w < 2 * NB; ++w) {
    if (w < wave) v += sred[w][0];
    K += sred[w][1];
  }
  v += K;
  float pa = 0.f, pd = 0.f;
  if (tid < Q) {
    if (t < nv) ddt[(r0 + t) * H + h] = f32_to_bf16(sdsv + Ah * v);
    pa = dtv * v;
    pd = ddv;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    pa += __shfl_xor(pa, off, 64);
    pd += __shfl_xor(pd, off, 64);
  }
  __syncthreads();
  if (lane == 0) {
    sred[wave][0] = pa;
    sred[wave][1] = pd;
  }
  __syncthreads();
  if (tid == 0) {
    float a = 0.f, d = 0.f;
    for (int w = 0; w < 2 * NB; ++w) {
      a += sred[w][0];
      d += sred[w][1];
    }
    dAp[((size_t(b) * H + h) * nc + c)] = a;
    dDp[((size_t(b) * H + h) * nc + c)] = d;
  }
}

// dB, dC: sum over the heads of each group of the per-head fp32 partials
// (fixed order), rounded to bf16; dA, dD: sums over batch rows and chunks.
__global__ __launch_bounds__(256) void bwd_reduce_bc(const float* __restrict__ dBp, const float* __restrict__ dCp,
                                                     uint16_t* __restrict__ dB, uint16_t* __restrict__ dC,
                                                     long rows, int H, int G, int N) {
  const long e = long(blockIdx.x) * 256 + threadIdx.x;   // (row, group, 4 n)
  const int n4 = N / 4;
  if (e >= rows * G * n4) return;
  const int nq = int(e % n4);
  const long rg = e / n4;
  const int g = int(rg % G);
  const long row = rg / G;
  const int hpg = H / G;
  f32x4 sb = f32x4{0.f, 0.f, 0.f, 0.f}, sc = sb;
  for (int k = 0; k < hpg; ++k) {
    const size_t o = (size_t(row) * H + g * hpg + k) * N + 4 * nq;
    const f32x4 vb = *reinterpret_cast<const f32x4*>(dBp + o);
    const f32x4 vc = *reinterpret_cast<const f32x4*>(dCp + o);
    sb += vb;
    sc += vc;
  }
  const size_t oo = (size_t(row) * G + g) * N + 4 * nq;
  *reinterpret_cast<u32x2*>(dB + oo) = u32x2{pack_bf16x2(sb[0], sb[1]), pack_bf16x2(sb[2], sb[3])};
  *reinterpret_cast<u32x2*>(dC + oo) = u32x2{pack_bf16x2(sc[0], sc[1]), pack_bf16x2(sc[2], sc[3])};
}

__global__ __launch_bounds__(64) void bwd_reduce_ad(const float* __restrict__ dAp, const float* __restrict__ dDp,
                                                    float* __restrict__ dA, float* __restrict__ dD, int batch,
                                                    int H, int nc) {
  const int h = blockIdx.x;
  float a = 0.f, d = 0.f;
  for (long k = threadIdx.x; k < long(batch) * nc; k += 64) {
    const int bb = int(k / nc), cc = int(k % nc);
    a += dAp[(size_t(bb) * H + h) * nc + cc];
    d += dDp[(size_t(bb) * H + h) * nc + cc];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    a += __shfl_xor(a, off, 64);
    d += __shfl_xor(d, off, 64);
  }
  if (threadIdx.x == 0) {
    dA[h] = a;
    if (dD) dD[h] = d;
  }
}

template <int N, int P, int NB>
hipError_t launch_npq(const FwdShape& s, const BwdArgs& a, hipStream_t st) {
  const long blocks = long(s.b) * s.nc * s.H;
  hipLaunchKernelGGL((bwd_chunk_kernel<N, P, NB>), dim3(unsigned(blocks)), dim3(128 * NB), 0, st,
                     static_cast<const uint16_t*>(a.x), static_cast<const uint16_t*>(a.B),
                     static_cast<const uint16_t*>(a.C), static_cast<const uint16_t*>(a.dy), a.Acs, a.dtq, a.CB, a.CBt,
                     a.Hst, a.Gb, a.GbT, a.ghp, a.A, a.D, static_cast<uint16_t*>(a.dx), static_cast<uint16_t*>(a.ddt),
                     a.dBp, a.dCp, a.dAp, a.dDp, s.T, s.H, s.G, s.nc, a.nghp);
  return hipGetLastError();
}

template <int N, int P>
hipError_t launch_np(const FwdShape& s, const BwdArgs& a, hipStream_t st) {
  constexpr int Qb = bwd_chunk_len(P, N);     // one kernel per (dstate, headdim)
  if constexpr (Qb >= 32) return launch_npq<N, P, Qb / 32>(s, a, st);
  return hipErrorInvalidValue;
}

template <int N>
hipError_t launch_n(const FwdShape& s, const BwdArgs& a, hipStream_t st) {
  switch (s.P) {
    case 32: return launch_np<N, 32>(s, a, st);
    case 64: return launch_np<N, 64>(s, a, st);
    case 128: return launch_np<N, 128>(s, a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd_chunk(const FwdShape& s, const BwdArgs& a, hipStream_t st) {
  if (s.Q != bwd_chunk_len(s.P, s.N)) return hipErrorInvalidValue;
  switch (s.N) {
    case 32: return launch_n<32>(s, a, st);
    case 64: return launch_n<64>(s, a, st);
    case 128: return launch_n<128>(s, a, st);
    case 256: return launch_n<256>(s, a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_reduce(const FwdShape& s, const float* dBp, const float* dCp, const float* dAp,
                             const float* dDp, void* dB, void* dC, float* dA, float* dD, hipStream_t st) {
  const long rows = long(s.b) * s.T;
  const long n = rows * s.G * (s.N / 4);
  hipLaunchKernelGGL(bwd_reduce_bc, dim3(unsigned((n + 255) / 256)), dim3(256), 0, st, dBp, dCp,
                     static_cast<uint16_t*>(dB), static_cast<uint16_t*>(dC), rows, s.H, s.G, s.N);
  hipLaunchKernelGGL(bwd_reduce_ad, dim3(unsigned(s.H)), dim3(64), 0, st, dAp, dDp, dA, dD, s.b, s.H, s.nc);
  return hipGetLastError();
}

}  // namespace ssd
