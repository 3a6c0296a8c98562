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
// The decay exponents get
//   dAcs_t = C_t . dC_t - dt_t (B_t . dB'_t) + [t = Q-1] <G_c, H_{c+1}>
// and, since Acs_t = A sum_{k<=t} dt_k,
//   ddt_t = B_t . dB'_t + A R_t,  dA = sum_t dt_t R_t,  R_t = sum_{t'>=t} dAcs_t'.
//
// Precision of R. The in-chunk parts of C_t . dC_t and B_t . dB'_t are the
// row and column sums of W_ls = (C_l . B_s) e_ls Sxy_sl (dt_s W_ls over s;
// W_ls over l), which cancel in R except on the cross block s < t <= l, so
// both are taken in fp32 from the same fp32 products (fp32 C B^T tiles from
// the recomputation), never from the bf16 operands of the dB / dC products.
// Likewise H_c enters the dot C_l . (state term of dC_l) as a bf16 pair
// hi + lo. And with H_{c+1} = exp(Acs_{Q-1}) H_c + sum_s e_{Q-1,s} dt_s B_s x_s^T,
//   <G_c, H_{c+1}> = exp(Acs_{Q-1}) <G_c, H_c> + sum_s dt_s B_s . (e_{Q-1,s} G_c x_s)
// is formed from the same per-token state dots that the second term of
// dAcs subtracts, so those cancel exactly as well.
//
// dB and dC sum over the heads of a group: a work-group takes one (batch,
// chunk, group) and a slice of its heads, one head after the other, and keeps
// the sums in its accumulators (dt_s and the decays folded into the bf16
// operands), writing bf16 when it holds the whole group, else an fp32 partial
// per slice that a last kernel adds in a fixed order (as dA, dD over chunks).
//
// Two kernels: one work-group per (batch, chunk, group, slice of heads) with
// the s side (dx, dB; wave i owns 32-token block i as the tokens s and the
// tiles of l-blocks j >= i) and the l side (dC; wave NB + i owns block i as
// the tokens l and the tiles of s-blocks j <= i), and a last one per (batch,
// chunk, head) that turns the per-token dots of both into ddt, dA and dD. The s side works in tiles whose lanes are tokens s
// (registers over rows l), so its two contractions over l take the tile as
// the B operand under the k permutation the A operand reproduces with
// transposed LDS reads (as chunk_scan does); the l side mirrors it with
// lanes = l. Every decay factor has a non-positive exponent (off the
// diagonal split at a block boundary, on it masked).
#include <type_traits>

#include "mfma_util.h"

namespace ssd {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Element offset, in a ROWS-swizzled natural tile with RB chunks per row, of
// lane `lane`'s 8-byte transposed read u (0, 1) of the 32-column block mt:
// rows 4 (lane/32) + 8 u + (lane%16)/4 of a 32-row block whose k order is the
// accumulator row order, columns 32 mt + 16 ((lane/16)%2) + 4 (lane%4) .. +3.
template <int RB>
__device__ __forceinline__ int tr_off(int lane, int u, int mt) {
  const int q16 = lane & 15;
  return lds_off<RB, true>(4 * (lane >> 5) + 8 * u + (q16 >> 2), 32 * mt + 16 * ((lane >> 4) & 1) + 4 * (q16 & 3));
}


// Rows 0 .. NROW-1 of a token-major tensor (row stride `stride` elements,
// RB 16-byte chunks from `col0`) of the chunk, into registers (rows past the
// valid tokens as zeros) and then into a swizzled natural LDS tile. All
// threads of the work-group take part; the loads of several tensors are
// issued together before any store, so one round trip covers them all.
template <int RB, int NROW, int kThr>
struct RowStage {
  static constexpr int PER = (NROW * RB + kThr - 1) / kThr;
  static constexpr bool kEven = NROW * RB % kThr == 0;   // every thread takes PER chunks
  u32x4 v[PER];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, long r0, int nv, size_t stride,
                                       size_t col0, int tid) {
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int e = tid + m * kThr;
      const int r = e / RB, cc = e % RB;
      if (kEven || e < NROW * RB)
        v[m] = keep_or_zero(r < nv, load16(src + (r0 + min(r, nv - 1)) * stride + col0 + 8 * cc));
    }
  }
  template <bool ROWS>
  __device__ __forceinline__ void store(uint16_t* tile, int tid) const {
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int e = tid + m * kThr;
      if (kEven || e < NROW * RB) *reinterpret_cast<u32x4*>(&tile[lds_off<RB, ROWS>(e / RB, 8 * (e % RB))]) = v[m];
    }
  }
};

// 16 bytes (8 consecutive columns from col) of row r of a swizzled natural tile
// (tiles read by rows use the ROWS swizzle of mfma_util.h: 32 lanes reading
// one chunk column of 32 rows hit 2-way bank conflicts instead of 8-way)
template <int RB>
__device__ __forceinline__ u32x4 lds_row16(const uint16_t* tile, int r, int col) {
  return *reinterpret_cast<const u32x4*>(&tile[lds_off<RB, true>(r, col)]);
}
template <int RB>
__device__ __forceinline__ u32x2 lds_row8(const uint16_t* tile, int r, int col) {
  return *reinterpret_cast<const u32x2*>(&tile[lds_off<RB, true>(r, col)]);
}

// The s and l sides of one (batch, chunk, group) and a slice of the group's
// heads, in one work-group of 2 NB waves. Waves 0 .. NB-1 take the s side of
// 32-token block i = wave: dx, dB (summed over the heads) and, per head and
// token s, B_s . dB'_s (sds), dt_s B_s . (e_{Q-1,s} G_c x_s) (sdst) and
// dy_s . x_s (sdd), over the tiles of l-blocks j >= i. Waves NB .. 2NB-1 take
// the l side of block i = wave - NB: dC (summed over the heads) and, per head
// and token l, C_l . dC_l (sdl), over the tiles of s-blocks j <= i. Block i
// has NB - i tiles on the s side and i + 1 on the l side: waves w and w + NB,
// which the round-robin placement of a work-group's waves puts on one SIMD,
// hold NB + 1 tiles together on every SIMD. The chunk's B and C rows are
// staged once per work-group, each head's x, dy, G_c and bf16(H_c) once per
// head for both sides (all tiles in the ROWS swizzle except bf16(H_c), which
// is read transposed only); the fp32 C B^T tiles come from memory one tile
// ahead, and the hi + lo pair of H_c for the l side's dot straight from its
// fp32 rows.
template <int N, int P, int NB>
__global__ __launch_bounds__(128 * NB) void bwd_sl_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const uint16_t* __restrict__ dy, const float* __restrict__ Acs, const float* __restrict__ dtq,
    const float* __restrict__ CBf, const float* __restrict__ CBt, const float* __restrict__ Hst,
    const uint16_t* __restrict__ Gb, const float* __restrict__ D, uint16_t* __restrict__ dx,
    uint16_t* __restrict__ dBo, uint16_t* __restrict__ dCo, float* __restrict__ dBs, float* __restrict__ dCs,
    float* __restrict__ gsds, float* __restrict__ gsdst, float* __restrict__ gsdd, float* __restrict__ gsdl,
    int T, int H, int G, int nc, int nslice) {
  constexpr int Q = 32 * NB;
  constexpr int kThr = 128 * NB;
  constexpr int RBP = P / 8, RBN = N / 8;   // 16-byte chunks per row
  constexpr int ntile = NB * (NB + 1) / 2;
  __shared__ __attribute__((aligned(16))) uint16_t sB[Q * N];
  __shared__ __attribute__((aligned(16))) uint16_t sC[Q * N];
  __shared__ __attribute__((aligned(16))) uint16_t sX[Q * P];
  __shared__ __attribute__((aligned(16))) uint16_t sDY[Q * P];
  __shared__ __attribute__((aligned(16))) uint16_t sG[P * N];     // G_c, rows p
  // the state's low part in LDS too where it fits beside the rest (else the
  // C . dC dot reads H_c's fp32 rows from memory)
  constexpr bool HLO = bwd_lds_bytes(P, N, Q) + 2L * P * N <= kBwdLdsMax;
  __shared__ __attribute__((aligned(16))) uint16_t sH[P * N];     // bf16(H_c) = hi, rows p
  __shared__ __attribute__((aligned(16))) uint16_t sHl[HLO ? P * N : 8];   // bf16(H_c - hi) = lo
  __shared__ float sA2[Q], sdt[Q], sEL[Q], sEl[Q], sF[Q], sL[Q];

  const int id = xcd_swizzle(blockIdx.x, gridDim.x);
  const int sl = id % nslice;
  const int rest = id / nslice;
  const int g = rest % G;
  const int bc = rest / G;
  const int c = bc % nc, b = bc / nc;
  const int hps = H / G / nslice;               // heads of this work-group
  const int h0 = g * (H / G) + sl * hps;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_id();
  const bool sside = wave < NB;
  const int i = sside ? wave : wave - NB;       // this wave's 32-token block
  const int l32 = lane & 31, g2 = lane >> 5;
  const long r0 = long(b) * T + long(c) * Q;        // first token row of the chunk
  const int nv = min(Q, T - c * Q);                 // valid tokens

  {
    RowStage<RBN, Q, kThr> rb, rc;
    rb.load(Bm, r0, nv, size_t(G) * N, size_t(g) * N, tid);
    rc.load(Cm, r0, nv, size_t(G) * N, size_t(g) * N, tid);
    rb.template store<true>(sB, tid);
    rc.template store<true>(sC, tid);
  }
  // the chunk's tiles, [tile][4][64 lanes] float4; this lane's first quad
  const size_t tbase = ((size_t(b) * nc + c) * G + g) * size_t(ntile) * 1024;
  const f32x4* tS = reinterpret_cast<const f32x4*>(CBt + tbase) + lane;   // lanes = s
  const f32x4* tL = reinterpret_cast<const f32x4*>(CBf + tbase) + lane;   // lanes = l


  // dB (s side) or dC (l side) of this wave's 32 tokens summed over the
  // work-group's heads: transposed, rows n, lane = token
  f32x16 accT[N / 32];
#pragma unroll
  for (int nt = 0; nt < N / 32; ++nt) accT[nt] = zero16();

  for (int hk = 0; hk < hps; ++hk) {
    const int h = h0 + hk;
    const size_t arow = ((size_t(b) * H + h) * nc + c) * Q;
    const size_t sbase = ((size_t(b) * nc + c) * H + h) * size_t(P) * N;
    // lane constants, recomputed per head (see opaque)
    const int tid = opaque(threadIdx.x), lane = tid & 63;
    const int l32 = lane & 31, g2 = lane >> 5;
    __syncthreads();   // the previous head's tiles and tables are consumed
    {
    // the head's operands: its decay tables (thread t < Q takes token t), x
    // and dy rows, G_c and H_c, loaded by all threads together
    constexpr int PH = (P * RBN + kThr - 1) / kThr;
    constexpr bool kHEven = P * RBN % kThr == 0;
    RowStage<RBP, Q, kThr> rx, rd;
    RowStage<RBN, P, kThr> rg;
    f32x4 hv[PH][2];
    float ta = 0.f, tbs = 0.f, tbl = 0.f, tc = 0.f, td = 0.f;
    if (tid < Q) {
      ta = Acs[arow + tid];
      tbs = Acs[arow + (tid & ~31)];
      tbl = Acs[arow + (tid | 31)];
      tc = Acs[arow + Q - 1];
      td = dtq[arow + tid];
    }
    rx.load(x, r0, nv, size_t(H) * P, size_t(h) * P, tid);
    rd.load(dy, r0, nv, size_t(H) * P, size_t(h) * P, tid);
    rg.load(Gb + sbase, 0, P, N, 0, tid);
#pragma unroll
    for (int m = 0; m < PH; ++m) {
      const int e = tid + m * kThr;
      if (kHEven || e < P * RBN) {
        const float* hr = Hst + sbase + size_t(e / RBN) * N + 8 * (e % RBN);
        hv[m][0] = *reinterpret_cast<const f32x4*>(hr);
        hv[m][1] = *reinterpret_cast<const f32x4*>(hr + 4);
      }
    }
    if (tid < Q) {
      const float a2 = ta * kLog2e;
      sA2[tid] = a2;
      sdt[tid] = td;
      sEL[tid] = __builtin_amdgcn_exp2f(a2 - tbs * kLog2e);         // <= 1
      sEl[tid] = __builtin_amdgcn_exp2f(tc * kLog2e - a2);          // <= 1
      sF[tid] = __builtin_amdgcn_exp2f(tbl * kLog2e - a2) * td;     // <= dt
      sL[tid] = __builtin_amdgcn_logf(td) - a2;                     // -inf where dt = 0
    }
    rx.template store<true>(sX, tid);
    rd.template store<true>(sDY, tid);
    rg.template store<true>(sG, tid);
#pragma unroll
    for (int m = 0; m < PH; ++m) {
      const int e = tid + m * kThr;
      if (kHEven || e < P * RBN) {
        // H_c as the bf16 pair hi + lo (lo = bf16(H - hi)): hi alone is the
        // operand of the dC state term, the pair the one of the C . dC dot
        u32x4 hi, lo;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float v0 = hv[m][w / 2][2 * (w % 2)], v1 = hv[m][w / 2][2 * (w % 2) + 1];
          hi[w] = pack_bf16x2(v0, v1);
          lo[w] = pack_bf16x2(v0 - bf16_lo(hi[w]), v1 - bf16_hi(hi[w]));
        }
        const int o = lds_off<RBN, true>(e / RBN, 8 * (e % RBN));
        *reinterpret_cast<u32x4*>(&sH[o]) = hi;
        if constexpr (HLO) *reinterpret_cast<u32x4*>(&sHl[o]) = lo;
      }
    }
    }
    __syncthreads();

    if (sside) {
      // ------------------------------------------------------------ s side
      const int s = 32 * i + l32;
      const bool sok = s < nv;
      const long srow = r0 + min(s, nv - 1);
      const int jend = min(NB, (nv + 31) / 32);   // l-blocks past the valid tokens add nothing

      const float dts = sdt[s], a2s = sA2[s], els = sEl[s];
      u32x4 xr[P / 16];
#pragma unroll
      for (int kk = 0; kk < P / 16; ++kk) xr[kk] = lds_row16<RBP>(sX, s, 16 * kk + 8 * g2);

      // state terms. dx^T(p, s) = e_{Q-1,s} dt_s sum_n G(n, p) B_s[n]; the same
      // product dotted with x_s is this head's B_s . (e_{Q-1,s} G_c x_s)
      f32x16 adx[P / 32];
#pragma unroll
      for (int pt = 0; pt < P / 32; ++pt) {
        adx[pt] = zero16();
#pragma unroll
        for (int kk = 0; kk < N / 16; ++kk)
          adx[pt] = mfma32x32x16(lds_row16<RBN>(sG, 32 * pt + l32, 16 * kk + 8 * g2),
                                 lds_row16<RBN>(sB, s, 16 * kk + 8 * g2), adx[pt]);
      }
      float bdst = 0.f;
#pragma unroll
      for (int pt = 0; pt < P / 32; ++pt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2 xv = lds_row8<RBP>(sX, s, 32 * pt + 8 * q + 4 * g2);
          bdst += adx[pt][4 * q] * bf16_lo(xv[0]) + adx[pt][4 * q + 1] * bf16_hi(xv[0]) +
                  adx[pt][4 * q + 2] * bf16_lo(xv[1]) + adx[pt][4 * q + 3] * bf16_hi(xv[1]);
#pragma unroll
          for (int r = 0; r < 4; ++r) adx[pt][4 * q + r] *= dts * els;
        }
      bdst = els * (bdst + __shfl_xor(bdst, 32, 64));
      // dB^T(n, s) += sum_p G(n, p) (dt_s e_{Q-1,s} x_s[p])   (G rows n: transposed reads)
      {
        u32x4 xs[P / 16];
        const float f = dts * els;
#pragma unroll
        for (int kk = 0; kk < P / 16; ++kk)
#pragma unroll
          for (int w = 0; w < 4; ++w) xs[kk][w] = pack_bf16x2(bf16_lo(xr[kk][w]) * f, bf16_hi(xr[kk][w]) * f);
#pragma unroll
        for (int nt = 0; nt < N / 32; ++nt)
#pragma unroll
          for (int kk = 0; kk < P / 16; ++kk) {
            const int kb = 16 * kk + 8 * g2;
            accT[nt] = mfma32x32x16(frag_tr<RBN, true>(sG, kb, kb + 4, 32 * nt, lane), xs[kk], accT[nt]);
          }
      }

      // dy_s . x_s (for dD)
      float dd = 0.f;
#pragma unroll
      for (int kk = 0; kk < P / 16; ++kk) {
        const u32x4 dv = lds_row16<RBP>(sDY, s, 16 * kk + 8 * g2);
#pragma unroll
        for (int w = 0; w < 4; ++w)
          dd += bf16_lo(dv[w]) * bf16_lo(xr[kk][w]) + bf16_hi(dv[w]) * bf16_hi(xr[kk][w]);
      }
      dd += __shfl_xor(dd, 32, 64);
      // intra-chunk terms, one 32 x 32 tile (rows l of block j, lanes s) at a time
      float bd = 0.f;                              // this head's sum_l W_ls
      // one tile; the diagonal one (j == i, masked) apart from the others
      auto tile = [&](int j, auto diag_c) {
        constexpr bool diag = decltype(diag_c)::value;
        const int ln = opaque(lane);                 // per-tile addresses (see opaque)
        // C_l . B_s, rows l in accumulator order (from L2; used after the Sxy products)
        const f32x4* tp = tS + (j * (j + 1) / 2 + i) * 256;
        const f32x4 cb4[4] = {tp[0], tp[64], tp[128], tp[192]};
        f32x16 accS = zero16();
#pragma unroll
        for (int kk = 0; kk < P / 16; ++kk)
          accS = mfma32x32x16(lds_row16<RBP>(sDY, 32 * j + (ln & 31), 16 * kk + 8 * (ln >> 5)),
                              lds_row16<RBP>(sX, 32 * i + (ln & 31), 16 * kk + 8 * (ln >> 5)), accS);   // Sxy^T
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
            if constexpr (diag) {
              const float ex = __builtin_amdgcn_exp2f(fminf(sA2[l] - a2s, 0.f));
              e2[u] = l >= s ? ex : 0.f;
            } else {
              e2[u] = sEL[l] * lf;
            }
          }
          const float z0 = e2[0] * accS[2 * m], z1 = e2[1] * accS[2 * m + 1];
          bd += z0 * cb_lo + z1 * cb_hi;                              // column sum of W
          zw[m] = pack_bf16x2(dts * z0, dts * z1);
          mw[m] = pack_bf16x2(e2[0] * dts * cb_lo, e2[1] * dts * cb_hi);
        }
        const u32x4 zga = u32x4{zw[0], zw[1], zw[2], zw[3]}, zgb = u32x4{zw[4], zw[5], zw[6], zw[7]};
        const u32x4 mga = u32x4{mw[0], mw[1], mw[2], mw[3]}, mgb = u32x4{mw[4], mw[5], mw[6], mw[7]};
        // dx^T(p, s) += sum_l dy^T(p, l) M(l, s)
        const int joP = 32 * j * P;
#pragma unroll
        for (int pt = 0; pt < P / 32; ++pt) {
          const int o0 = tr_off<RBP>(ln, 0, pt) + joP, o1 = tr_off<RBP>(ln, 1, pt) + joP;
          const u32x2 a0 = lds_read_tr16(sDY, o0), a1 = lds_read_tr16(sDY, o1);
          const u32x2 b0 = lds_read_tr16(sDY, o0 + 16 * P), b1 = lds_read_tr16(sDY, o1 + 16 * P);
          adx[pt] = mfma32x32x16(u32x4{a0[0], a0[1], a1[0], a1[1]}, mga, adx[pt]);
          adx[pt] = mfma32x32x16(u32x4{b0[0], b0[1], b1[0], b1[1]}, mgb, adx[pt]);
        }
        // dB^T(n, s) += sum_l C^T(n, l) dt_s Z(l, s)
        const int joN = 32 * j * N;
#pragma unroll
        for (int nt = 0; nt < N / 32; ++nt) {
          const int o0 = tr_off<RBN>(ln, 0, nt) + joN, o1 = tr_off<RBN>(ln, 1, nt) + joN;
          const u32x2 a0 = lds_read_tr16(sC, o0), a1 = lds_read_tr16(sC, o1);
          const u32x2 b0 = lds_read_tr16(sC, o0 + 16 * N), b1 = lds_read_tr16(sC, o1 + 16 * N);
          accT[nt] = mfma32x32x16(u32x4{a0[0], a0[1], a1[0], a1[1]}, zga, accT[nt]);
          accT[nt] = mfma32x32x16(u32x4{b0[0], b0[1], b1[0], b1[1]}, zgb, accT[nt]);
        }
      };
      if (i < jend) tile(i, std::true_type{});
      for (int j = i + 1; j < jend; ++j) tile(j, std::false_type{});

      // dx = ... + D dy (rows p = 32 pt + 8 q + 4 g2 + 0..3 of lane s), stored as bf16
      const float Dh = D ? D[h] : 0.f;
#pragma unroll
      for (int pt = 0; pt < P / 32; ++pt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int p = 32 * pt + 8 * q + 4 * g2;
          const u32x2 dv = lds_row8<RBP>(sDY, s, p);
          const float v0 = adx[pt][4 * q] + Dh * bf16_lo(dv[0]), v1 = adx[pt][4 * q + 1] + Dh * bf16_hi(dv[0]);
          const float v2 = adx[pt][4 * q + 2] + Dh * bf16_lo(dv[1]), v3 = adx[pt][4 * q + 3] + Dh * bf16_hi(dv[1]);
          if (sok)
            *reinterpret_cast<u32x2*>(dx + (srow * H + h) * size_t(P) + p) =
                u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
        }
      bd += __shfl_xor(bd, 32, 64);
      if (g2 == 0) {
        gsds[arow + s] = sok ? bd + bdst : 0.f;     // B_s . dB'_s of this head
        gsdst[arow + s] = sok ? dts * bdst : 0.f;
        gsdd[arow + s] = dd;
      }
    } else {
      // ------------------------------------------------------------ l side
      const int l = 32 * i + l32;
      const bool lok = l < nv;
      const int jlast = 32 * i < nv ? i : -1;       // no tiles when the whole block is past the tokens

      const float a2l = sA2[l];
      const float el = __builtin_amdgcn_exp2f(a2l);
      u32x4 dyr[P / 16];
#pragma unroll
      for (int kk = 0; kk < P / 16; ++kk) dyr[kk] = lds_row16<RBP>(sDY, l, 16 * kk + 8 * g2);
      // state term of dC: dC^T(n, l) += sum_p H(n, p) (exp(Acs_l) dy_l[p])
      {
        u32x4 dys[P / 16];
#pragma unroll
        for (int kk = 0; kk < P / 16; ++kk)
#pragma unroll
          for (int w = 0; w < 4; ++w) dys[kk][w] = pack_bf16x2(bf16_lo(dyr[kk][w]) * el, bf16_hi(dyr[kk][w]) * el);
#pragma unroll
        for (int nt = 0; nt < N / 32; ++nt)
#pragma unroll
          for (int kk = 0; kk < P / 16; ++kk) {
            const int kb = 16 * kk + 8 * g2;
            accT[nt] = mfma32x32x16(frag_tr<RBN, true>(sH, kb, kb + 4, 32 * nt, lane), dys[kk], accT[nt]);
          }
      }
      // this head's C_l . (state term of dC_l) = exp(Acs_l) dy_l . (H^T C_l),
      // with H as hi + lo (rows p): y^T(p, l) = sum_n H(n, p) C_l[n]
      float cd = 0.f;
      {
        f32x16 yst[P / 32];
#pragma unroll
        for (int pt = 0; pt < P / 32; ++pt) {
          const float* hrow = Hst + sbase + size_t(32 * pt + l32) * N + 8 * g2;
          yst[pt] = zero16();
#pragma unroll 2
          for (int kk = 0; kk < N / 16; ++kk) {
            const u32x4 cl = lds_row16<RBN>(sC, l, 16 * kk + 8 * g2);
            u32x4 hi, lo;
            if constexpr (HLO) {
              hi = lds_row16<RBN>(sH, 32 * pt + l32, 16 * kk + 8 * g2);
              lo = lds_row16<RBN>(sHl, 32 * pt + l32, 16 * kk + 8 * g2);
            } else {
              const f32x4 hq0 = *reinterpret_cast<const f32x4*>(hrow + 16 * kk);
              const f32x4 hq1 = *reinterpret_cast<const f32x4*>(hrow + 16 * kk + 4);
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                const f32x4& hq = w < 2 ? hq0 : hq1;
                const float v0 = hq[2 * (w % 2)], v1 = hq[2 * (w % 2) + 1];
                hi[w] = pack_bf16x2(v0, v1);
                lo[w] = pack_bf16x2(v0 - bf16_lo(hi[w]), v1 - bf16_hi(hi[w]));
              }
            }
            yst[pt] = mfma32x32x16(hi, cl, yst[pt]);
            yst[pt] = mfma32x32x16(lo, cl, yst[pt]);
          }
        }
#pragma unroll
        for (int pt = 0; pt < P / 32; ++pt)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x2 dv = lds_row8<RBP>(sDY, l, 32 * pt + 8 * q + 4 * g2);
            cd += yst[pt][4 * q] * bf16_lo(dv[0]) + yst[pt][4 * q + 1] * bf16_hi(dv[0]) +
                  yst[pt][4 * q + 2] * bf16_lo(dv[1]) + yst[pt][4 * q + 3] * bf16_hi(dv[1]);
          }
        cd *= el;
      }
      // intra-chunk terms, tiles of rows s (block j) and lanes l
      // one tile; the diagonal one (j == i, masked) apart from the others
      auto tile = [&](int j, auto diag_c) {
        constexpr bool diag = decltype(diag_c)::value;
        const int ln = opaque(lane);                 // per-tile addresses (see opaque)
        // C B^T in the forward orientation (rows s, lane l)
        const f32x4* tp = tL + (i * (i + 1) / 2 + j) * 256;
        const f32x4 cf4[4] = {tp[0], tp[64], tp[128], tp[192]};
        f32x16 accS = zero16();
#pragma unroll
        for (int kk = 0; kk < P / 16; ++kk)
          accS = mfma32x32x16(lds_row16<RBP>(sX, 32 * j + (ln & 31), 16 * kk + 8 * (ln >> 5)),
                              lds_row16<RBP>(sDY, 32 * i + (ln & 31), 16 * kk + 8 * (ln >> 5)), accS);   // Sxy
        const float lfac = diag ? 0.f : __builtin_amdgcn_exp2f(a2l - sA2[32 * j + 31]);
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
            if constexpr (diag) {
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
          const int o0 = tr_off<RBN>(ln, 0, nt) + joN, o1 = tr_off<RBN>(ln, 1, nt) + joN;
          const u32x2 a0 = lds_read_tr16(sB, o0), a1 = lds_read_tr16(sB, o1);
          const u32x2 b0 = lds_read_tr16(sB, o0 + 16 * N), b1 = lds_read_tr16(sB, o1 + 16 * N);
          accT[nt] = mfma32x32x16(u32x4{a0[0], a0[1], a1[0], a1[1]}, zga, accT[nt]);
          accT[nt] = mfma32x32x16(u32x4{b0[0], b0[1], b1[0], b1[1]}, zgb, accT[nt]);
        }
      };
      for (int j = 0; j < jlast; ++j) tile(j, std::false_type{});
      if (jlast >= 0) tile(jlast, std::true_type{});
      cd += __shfl_xor(cd, 32, 64);
      if (g2 == 0) gsdl[arow + l] = lok ? cd : 0.f;   // C_l . dC_l of this head
    }
  }

  // ---- the work-group's sum over its heads: bf16 when it holds all heads
  //      of the group, else an fp32 partial of its slice
  const int t = 32 * i + l32;
  if (t < nv) {
    const size_t row = size_t(r0 + t) * G + g;
    const long rows = long(gridDim.x / nslice / G / nc) * T;   // batch rows x tokens
    uint16_t* out = sside ? dBo : dCo;
    float* part = sside ? dBs : dCs;
#pragma unroll
    for (int nt = 0; nt < N / 32; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = 32 * nt + 8 * q + 4 * g2;
        const f32x4 v4 = f32x4{accT[nt][4 * q], accT[nt][4 * q + 1], accT[nt][4 * q + 2], accT[nt][4 * q + 3]};
        if (nslice == 1)
          *reinterpret_cast<u32x2*>(out + row * N + n) = u32x2{pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3])};
        else
          *reinterpret_cast<f32x4*>(part + (size_t(sl) * rows * G + row) * N + n) = v4;
      }
  }
}

// Last per-chunk step, one (batch, chunk, head) per work-group: dAcs, its
// reverse cumulative sum R, ddt and the chunk's dA / dD terms. Thread k < Q
// takes token t = Q-1-k, so an inclusive scan over k is the sum over t' >= t.
// The chunk-end term (dAcs_{Q-1} only, so a constant K added to every R_t)
// is a block sum: the per-token state dots and exp(Acs_{Q-1}) <G_c, H_c>
// from the reverse pass's partials.
template <int Q>
__global__ __launch_bounds__(Q) void bwd_ddt_kernel(const float* __restrict__ Acs, const float* __restrict__ dtq,
                                                    const float* __restrict__ gsds, const float* __restrict__ gsdst,
                                                    const float* __restrict__ gsdd, const float* __restrict__ gsdl,
                                                    const float* __restrict__ ghp, const float* __restrict__ A,
                                                    uint16_t* __restrict__ ddt, float* __restrict__ dAp,
                                                    float* __restrict__ dDp, int T, int H, int nc, int nghp) {
  constexpr int kW = Q / 64 > 0 ? Q / 64 : 1;
  __shared__ float sred[kW][2];
  const int id = blockIdx.x;                     // (b * H + h) * nc + c
  const int c = id % nc, bh = id / nc;
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t arow = size_t(id) * Q;
  const int nv = min(Q, T - c * Q);
  const int t = Q - 1 - tid;
  const float dtv = dtq[arow + t], sdsv = gsds[arow + t];
  const float dacs = gsdl[arow + t] - dtv * sdsv;
  float kpart = gsdst[arow + t];
  for (int k = tid; k < nghp; k += Q)
    kpart += __builtin_amdgcn_exp2f(Acs[arow + Q - 1] * kLog2e) * ghp[size_t(id) * nghp + k];
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
  for (int w = 0; w < kW; ++w) {
    if (w < wave) v += sred[w][0];
    K += sred[w][1];
  }
  v += K;
  if (t < nv) ddt[(long(b) * T + long(c) * Q + t) * H + h] = f32_to_bf16(sdsv + A[h] * v);
  float pa = dtv * v, pd = gsdd[arow + t];
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
    for (int w = 0; w < kW; ++w) {
      a += sred[w][0];
      d += sred[w][1];
    }
    dAp[id] = a;
    dDp[id] = d;
  }
}

// dB, dC: sum of the per-slice fp32 partials (fixed order), rounded to bf16.
__global__ __launch_bounds__(256) void bwd_reduce_bc(const float* __restrict__ dBs, const float* __restrict__ dCs,
                                                     uint16_t* __restrict__ dB, uint16_t* __restrict__ dC,
                                                     long n4, int nslice) {
  const long e = long(blockIdx.x) * 256 + threadIdx.x;   // 4 elements of [b, T, G, N]
  if (e >= n4) return;
  f32x4 sb = f32x4{0.f, 0.f, 0.f, 0.f}, sc = sb;
  for (int k = 0; k < nslice; ++k) {
    sb += *reinterpret_cast<const f32x4*>(dBs + (size_t(k) * n4 + e) * 4);
    sc += *reinterpret_cast<const f32x4*>(dCs + (size_t(k) * n4 + e) * 4);
  }
  *reinterpret_cast<u32x2*>(dB + size_t(e) * 4) = u32x2{pack_bf16x2(sb[0], sb[1]), pack_bf16x2(sb[2], sb[3])};
  *reinterpret_cast<u32x2*>(dC + size_t(e) * 4) = u32x2{pack_bf16x2(sc[0], sc[1]), pack_bf16x2(sc[2], sc[3])};
}

// dA, dD: sums over batch rows and chunks of the per-(b, h, c) partials.
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
  const long blocks = long(s.b) * s.nc * s.G * a.nslice;
  hipLaunchKernelGGL((bwd_sl_kernel<N, P, NB>), dim3(unsigned(blocks)), dim3(128 * NB), 0, st,
                     static_cast<const uint16_t*>(a.x), static_cast<const uint16_t*>(a.B),
                     static_cast<const uint16_t*>(a.C), static_cast<const uint16_t*>(a.dy), a.Acs, a.dtq, a.CB,
                     a.CBt, a.Hst, a.Gb, a.D, static_cast<uint16_t*>(a.dx), static_cast<uint16_t*>(a.dB),
                     static_cast<uint16_t*>(a.dC), a.dBs, a.dCs, a.tsds, a.tsdst, a.tsdd, a.tsdl, s.T, s.H, s.G,
                     s.nc, a.nslice);
  hipLaunchKernelGGL((bwd_ddt_kernel<32 * NB>), dim3(unsigned(long(s.b) * s.H * s.nc)), dim3(32 * NB), 0, st,
                     a.Acs, a.dtq, a.tsds, a.tsdst, a.tsdd, a.tsdl, a.ghp, a.A, static_cast<uint16_t*>(a.ddt),
                     a.dAp, a.dDp, s.T, s.H, s.nc, a.nghp);
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

int bwd_slices(const FwdShape& s) {
  // heads of a group split over work-groups until the grid has a work-group
  // per compute unit of a 256-unit device (the per-chunk kernel's LDS allows
  // one per unit; slices divide the group's heads). Measured on the 130M
  // layer: 2 slices (256 work-groups) 0.314 ms per backward call, 4 slices
  // 0.330, 6 slices 0.342, 8 slices 0.354.
  const int hpg = s.H / s.G;
  const long base = long(s.b) * s.nc * s.G;
  for (int d = 1; d <= hpg; ++d)
    if (hpg % d == 0 && base * d >= 256) return d;
  return hpg;
}

hipError_t launch_bwd_chunk(const FwdShape& s, const BwdArgs& a, hipStream_t st) {
  if (s.Q != bwd_chunk_len(s.P, s.N) || a.nslice < 1 || (s.H / s.G) % a.nslice) return hipErrorInvalidValue;
  switch (s.N) {
    case 32: return launch_n<32>(s, a, st);
    case 64: return launch_n<64>(s, a, st);
    case 128: return launch_n<128>(s, a, st);
    case 256: return launch_n<256>(s, a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_reduce(const FwdShape& s, const BwdArgs& a, float* dA, float* dD, hipStream_t st) {
  if (a.nslice > 1) {
    const long n4 = long(s.b) * s.T * s.G * (s.N / 4);
    hipLaunchKernelGGL(bwd_reduce_bc, dim3(unsigned((n4 + 255) / 256)), dim3(256), 0, st, a.dBs, a.dCs,
                       static_cast<uint16_t*>(a.dB), static_cast<uint16_t*>(a.dC), n4, a.nslice);
  }
  hipLaunchKernelGGL(bwd_reduce_ad, dim3(unsigned(s.H)), dim3(64), 0, st, a.dAp, a.dDp, dA, dD, s.b, s.H, s.nc);
  return hipGetLastError();
}

}  // namespace ssd
