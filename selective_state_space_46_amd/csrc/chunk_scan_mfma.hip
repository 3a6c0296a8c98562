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
// Decay. For l, s in the same chunk, s <= l, the weight exp(Acs_l - Acs_s)
// dt_s is at most dt_s, but a product of per-token factors can overflow when
// one factor has a positive exponent (a factor exp(Acs_a - Acs_s) with s
// after a grows like exp(sum of dt |A|) over the span). Both factors used
// here have exponents <= 0:
//   s in an earlier 32-token column block that ends at token e:
//     exp(Acs_l - Acs_s) dt_s = exp(Acs_l - Acs_e) * [exp(Acs_e - Acs_s) dt_s]
//     the bracket depends on s only (a per-token table in LDS), the first
//     factor is one exponential per lane and tile;
//   s in the same 32-token block as l (the diagonal tile): one exponential
//     per element, exp(min(Acs_l - Acs_s, 0)) dt_s, masked to s <= l.
// Factors that underflow to zero stand for weights that are smaller still.
//
// Work-group: one batch row, one 256-token super-chunk (256/Q chunks), one
// head; 4 waves. The C B^T tiles come precomputed once per group
// (by the chunk_state launch, chunk_state_mfma.hip) in MFMA-fragment order. The super-chunk is cut into eight
// 32-row blocks l; wave w owns blocks w and 7-w so that the causal triangle
// splits evenly. The output is produced transposed (y^T: rows p, lane = token
// l), which makes every per-token factor one multiplier per lane:
//   1. y^T = H_c^T C_l^T (k = dstate): H_c^T staged once in LDS (bf16, from
//      state_passing) when the super-chunk is one chunk, C_l rows straight from
//      HBM; then y^T *= exp(Acs_l).
//   2. for each column block s <= l of the chunk: the C B^T tile (lane =
//      column l, registers = rows s in runs of 4) times the decay, rounded to
//      bf16, is the B operand of y^T += X^T G^T under a k permutation that the
//      X operand reproduces: x sits in LDS in natural token-major order
//      (swizzled 16-byte chunks) and is read transposed with
//      ds_read_b64_tr_b16. Tiles are loaded one tile ahead of use, into two
//      buffers used in turn.
//   3. + D x (x from the same LDS tile), bf16 rounding, 8-byte stores of 4
//      consecutive p.
#include "mfma_util.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kSC = 256;          // tokens per super-chunk
constexpr float kLog2e = 1.4426950408889634f;

// VARLEN: chunk rows from the chunk table tab (packed sequences), else the
// equal-length layout (tab unused).
template <int N, int P, bool HLDS, bool VARLEN>
__global__ __launch_bounds__(kThreads) void chunk_scan_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ CB, const uint16_t* __restrict__ Cm,
    const float* __restrict__ Acs, const float* __restrict__ dtq, const uint16_t* __restrict__ Hb,
    const float* __restrict__ D, uint16_t* __restrict__ y, const int4* __restrict__ tab, int T, int H,
    int G, int Q, int nc, int nsc) {
  constexpr int kHS = N + 8;  // H^T row stride (bf16): 16-byte reads of 16 lanes hit distinct banks
  constexpr int RBX = P / 8;  // 16-byte chunks per X' row
  constexpr int HROWS = HLDS ? P : 1;
  __shared__ __attribute__((aligned(16))) uint16_t sX[kSC * P];
  __shared__ __attribute__((aligned(16))) uint16_t sHt[HROWS][kHS];
  __shared__ __attribute__((aligned(16))) float sA[kSC];  // Acs * log2(e)
  __shared__ __attribute__((aligned(16))) float sF[kSC];  // exp(Acs[block end] - Acs_s) * dt_s
  __shared__ __attribute__((aligned(16))) float sL[kSC];  // log2(dt_s) - Acs_s log2(e)

  const int id = xcd_swizzle(blockIdx.x, gridDim.x);
  const int h = id % H;
  const int bs = id / H;
  const int sc = bs % nsc, b = bs / nsc;
  const int g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_id();  // wave-uniform (scalar register)
  const int l32 = lane & 31, g2 = lane >> 5;
  const int cps = kSC / Q;        // chunks per super-chunk
  const int c0 = sc * cps;        // first chunk of the super-chunk
  const int lpc = Q / 32;         // 32-row blocks per chunk
  const int ntile = lpc * (lpc + 1) / 2;
  // token rows of the super-chunk's chunks (ci = 0 .. cps-1); n = 0 past the last chunk
  auto crows = [&](int ci) {
    return c0 + ci < nc ? chunk_rows(VARLEN ? tab : static_cast<const int4*>(nullptr), b, c0 + ci, T, Q)
                        : ChunkRows{0, 0};
  };
  // fast: every row of the super-chunk is a valid token and the rows are
  // consecutive token rows (always so for equal-length batch rows);
  // rowsv: the first chunk with valid rows (a chunk table may leave any slot
  // unused)
  const ChunkRows rows0 = crows(0);
  ChunkRows rowsv = rows0;
  bool fast = true;
  for (int ci = 0; ci < cps; ++ci) {
    const ChunkRows r = crows(ci);
    fast = fast && r.n == Q && r.r0 == rows0.r0 + long(ci) * Q;
    if (rowsv.n <= 0) rowsv = r;
  }
  if (rowsv.n <= 0) return;            // no valid chunk: uniform, before any barrier

  // C B^T tiles of 32-row block i: tile jj (column block jfirst + jj) of the
  // block's row of its chunk's lower triangle, this lane's 32 bytes
  auto tile_src = [&](int i) {
    const int jf = (i / lpc) * lpc, cgi = c0 + i / lpc, ir = i - jf;
    return reinterpret_cast<const u32x4*>(
        CB + (((size_t(b) * nc + cgi) * G + g) * ntile + size_t(ir) * (ir + 1) / 2) * 1024 +
        size_t(lane) * 16);
  };
  // a block's first loads: its diagonal tile, its first tile, its C rows
  // (k = dstate, rows clamped into the tensor; zeroed past the end at use)
  auto issue_block_loads = [&](int i, u32x4 (&td)[2], u32x4 (&tn)[2], u32x4 (&cfv)[N / 16]) {
    const u32x4* ts = tile_src(i);
    const int ir = i - (i / lpc) * lpc;
    td[0] = ts[ir * 128];
    td[1] = ts[ir * 128 + 1];
    tn[0] = ts[0];
    tn[1] = ts[1];
    const ChunkRows r = crows(i / lpc);
    const long row = r.r0 + min((i % lpc) * 32 + l32, r.n - 1);
    const uint16_t* cr = Cm + (row * G + g) * size_t(N) + 8 * g2;
#pragma unroll
    for (int ks = 0; ks < N / 16; ++ks) cfv[ks] = load16(cr + 16 * ks);
  };
  u32x4 pre_tdiag[2], pre_tnext[2], pre_cf[N / 16];
  if ((wave % lpc) * 32 < crows(wave / lpc).n) issue_block_loads(wave, pre_tdiag, pre_tnext, pre_cf);

  // ---- staging 1: Acs, the per-token factor, H_c^T
  for (int i = tid; i < kSC; i += kThreads) {
    const int c = c0 + i / Q;
    float a = 0.f, f = 0.f, d = 0.f;
    if (crows(i / Q).n > 0) {
      const size_t row = ((size_t(b) * H + h) * nc + c) * Q;
      const int q = i % Q;
      a = Acs[row + q] * kLog2e;
      d = dtq[row + q];
      f = __builtin_amdgcn_exp2f(Acs[row + (q | 31)] * kLog2e - a) * d;  // exponent <= 0
    }
    sA[i] = a;
    sF[i] = f;
    sL[i] = __builtin_amdgcn_logf(d) - a;    // log2; -inf where dt = 0
  }
  if constexpr (HLDS) {
    const uint16_t* hsrc = Hb + ((size_t(b) * nc + c0) * H + h) * size_t(P) * N;
    static_assert(kThreads % (N / 8) == 0, "H staging shape");
    constexpr int kStep = kThreads / (N / 8);        // rows p per pass
    const int p0 = tid / (N / 8), seg = tid % (N / 8);
#pragma unroll
    for (int k = 0; k < (P + kStep - 1) / kStep; ++k)
      if (P % kStep == 0 || p0 + k * kStep < P)
        *reinterpret_cast<u32x4*>(&sHt[p0 + k * kStep][8 * seg]) =
            load16(hsrc + size_t(p0 + k * kStep) * N + 8 * seg);
  }
  // raw x, token-major, swizzled: issued with the loads above. Thread tid
  // copies 16-byte chunk tid % RBX of rows tid / RBX + k kStep; kStep is a
  // multiple of the swizzle period (16 rows), so every row of the thread has
  // the same swizzle and its LDS offsets differ by constants.
  static_assert(kThreads % RBX == 0 && (kThreads / RBX) % 16 == 0, "x staging shape");
  {
    constexpr int kStep = kThreads / RBX;
    const int r0 = tid / RBX, cc = tid % RBX;
    uint16_t* dst = &sX[lds_off<RBX, true>(r0, 8 * cc)];
    if (fast) {
      const uint16_t* src = x + ((rows0.r0 + r0) * H + h) * size_t(P) + 8 * cc;
      const size_t step = size_t(kStep) * H * P;
#pragma unroll
      for (int k = 0; k < RBX; ++k)
        *reinterpret_cast<u32x4*>(dst + k * kStep * P) = load16(src + k * step);
    } else {
#pragma unroll
      for (int k = 0; k < RBX; ++k) {
        const int r = r0 + k * kStep;
        const ChunkRows cr = crows(r / Q);
        const int rq = r % Q;
        // a chunk with no valid rows (past the last chunk, or an unused table
        // slot) reads a valid row of another chunk instead: any in-bounds row
        const long row = cr.n > 0 ? cr.r0 + min(rq, cr.n - 1) : rowsv.r0;
        const u32x4 v = load16(x + (row * H + h) * size_t(P) + 8 * cc);
        *reinterpret_cast<u32x4*>(dst + k * kStep * P) = keep_or_zero(rq < cr.n, v);
      }
    }
  }
  __syncthreads();

  // The transposed x reads of column block j start at row 32 j; the x tile's
  // swizzle repeats every 16 rows, so their addresses are lane constants (per
  // 32-column half pb and per 8-row half of a 16-row group) plus 32 j rows,
  // and the second fragment of a block sits 16 rows further.
  int xo[P / 32][2];
  {
    const int q16 = lane & 15;
    const int mcol = 16 * ((lane >> 4) & 1) + 4 * (q16 & 3);
#pragma unroll
    for (int pb = 0; pb < P / 32; ++pb)
#pragma unroll
      for (int u = 0; u < 2; ++u) xo[pb][u] = lds_off<RBX, true>(4 * g2 + 8 * u + (q16 >> 2), 32 * pb + mcol);
  }

  const float Dh = D ? D[h] : 0.f;
  for (int which = 0; which < 2; ++which) {
    const int i = which ? 7 - wave : wave;  // 32-row block of the super-chunk
    const ChunkRows cr = crows(i / lpc);
    const int rq0 = (i % lpc) * 32;         // first row of the block inside its chunk
    if (rq0 >= cr.n) continue;              // wave-uniform: nothing to produce
    const int jfirst = (i / lpc) * lpc;     // first column block of the same chunk
    const int cg = c0 + i / lpc;            // global chunk index (< nc)
    const int lcol = 32 * i + l32;          // this lane's output token in the super-chunk
    const int irel = i - jfirst;            // tiles of this block: jj = 0 .. irel
    const bool tok_ok = rq0 + l32 < cr.n;   // this lane's token is a valid one
    const long trow = cr.r0 + rq0 + l32;    // and its token row
    const u32x4* tsrc = tile_src(i);
    auto load_tile = [&](int jj, u32x4 (&tt)[2]) {
      tt[0] = tsrc[jj * 128];
      tt[1] = tsrc[jj * 128 + 1];
    };
    // this block's first loads: issued before the staging barrier for the
    // first block, here for the second
    u32x4 tdiag[2], tnext[2], cf[N / 16];
    if (which == 0) {
#pragma unroll
      for (int m = 0; m < 2; ++m) { tdiag[m] = pre_tdiag[m]; tnext[m] = pre_tnext[m]; }
#pragma unroll
      for (int ks = 0; ks < N / 16; ++ks) cf[ks] = pre_cf[ks];
    } else {
      issue_block_loads(i, tdiag, tnext, cf);
    }
    if (!fast) {
#pragma unroll
      for (int ks = 0; ks < N / 16; ++ks) cf[ks] = keep_or_zero(tok_ok, cf[ks]);
    }

    // ---- y^T = H_c^T C_l^T, then * exp(Acs_l)
    f32x16 acc[P / 32];
    const float sl = __builtin_amdgcn_exp2f(sA[lcol]);
#pragma unroll
    for (int pb = 0; pb < P / 32; ++pb) {
      acc[pb] = zero16();
#pragma unroll
      for (int ks = 0; ks < N / 16; ++ks) {
        u32x4 hf;
        if constexpr (HLDS) {
          hf = *reinterpret_cast<const u32x4*>(&sHt[32 * pb + l32][16 * ks + 8 * g2]);
        } else {
          hf = load16(Hb + (((size_t(b) * nc + cg) * H + h) * P + 32 * pb + l32) * size_t(N) + 16 * ks +
                      8 * g2);
        }
        acc[pb] = mfma32x32x16(hf, cf[ks], acc[pb]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[pb][r] *= sl;
    }

    // ---- y^T += X'^T G^T over the column blocks of the chunk
    const float al = sA[lcol];
    // one column block j: G^T = tile * decay (register pair m of the tile
    // holds rows s = 32 j + 8 (m/2) + 4 g2 + 2 (m%2) + {0, 1}), then two MFMAs
    // per 32 p. Off the diagonal (every s < every l) the decay is
    // exp(Acs_l - Acs_e) * [exp(Acs_e - Acs_s) dt_s] with e = 32 j + 31, the
    // column block's last token: both factors are <= 1. On the diagonal it is
    // exp(Acs_l - Acs_s) dt_s = 2^(Acs_l log2 e + [log2 dt_s - Acs_s log2 e])
    // per element (bracket from LDS; exponent <= log2 dt_s for s <= l), and
    // elements with s > l are replaced by zero, whatever their product.
    auto apply = [&](const int jj, const u32x4 (&tile)[2], const bool diag) {
      const int j = jfirst + jj;
      uint32_t gw[8];
      f32x4 fa[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        fa[q] = *reinterpret_cast<const f32x4*>(&(diag ? sL : sF)[32 * j + 8 * q + 4 * g2]);
      const float lfac = diag ? 0.f : __builtin_amdgcn_exp2f(al - sA[32 * j + 31]);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint32_t w = tile[m / 4][m % 4];
        const int k = 2 * (m % 2);
        float lo, hi;
        if (diag) {
          const int s0 = 8 * (m / 2) + 4 * g2 + k;
          const float plo = bf16_lo(w) * __builtin_amdgcn_exp2f(al + fa[m / 2][k]);
          const float phi = bf16_hi(w) * __builtin_amdgcn_exp2f(al + fa[m / 2][k + 1]);
          lo = s0 <= l32 ? plo : 0.f;
          hi = s0 + 1 <= l32 ? phi : 0.f;
        } else {
          lo = bf16_lo(w) * lfac * fa[m / 2][k];
          hi = bf16_hi(w) * lfac * fa[m / 2][k + 1];
        }
        gw[m] = pack_bf16x2(lo, hi);
      }
      const u32x4 ga = u32x4{gw[0], gw[1], gw[2], gw[3]};  // rows s = 32j + [0, 16)
      const u32x4 gb = u32x4{gw[4], gw[5], gw[6], gw[7]};  // rows s = 32j + [16, 32)
      const int jo = 32 * j * P;              // element offset of row 32 j (P elements per row)
#pragma unroll
      for (int pb = 0; pb < P / 32; ++pb) {
        const u32x2 a0 = lds_read_tr16(sX, xo[pb][0] + jo), a1 = lds_read_tr16(sX, xo[pb][1] + jo);
        const u32x2 b0 = lds_read_tr16(sX, xo[pb][0] + jo + 16 * P);
        const u32x2 b1 = lds_read_tr16(sX, xo[pb][1] + jo + 16 * P);
        acc[pb] = mfma32x32x16(u32x4{a0[0], a0[1], a1[0], a1[1]}, ga, acc[pb]);
        acc[pb] = mfma32x32x16(u32x4{b0[0], b0[1], b1[0], b1[1]}, gb, acc[pb]);
      }
    };
    // off-diagonal tiles two at a time, ping-pong buffers (the tile after
    // next loads while the current one is applied; no register copies)
    u32x4 tB[2];
    int jj = 0;
#pragma unroll 1
    for (; jj + 1 < irel; jj += 2) {
      load_tile(jj + 1, tB);
      apply(jj, tnext, false);
      if (jj + 2 < irel) load_tile(jj + 2, tnext);
      apply(jj + 1, tB, false);
    }
    if (jj < irel) apply(jj, tnext, false);
    apply(irel, tdiag, true);

    // ---- epilogue: + D x (x re-read, from L2), round, store 4 consecutive p (8 bytes) per run
    if (tok_ok) {
      u32x2 xr[P / 32][4];
#pragma unroll
      for (int pb = 0; pb < P / 32; ++pb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          xr[pb][q] = *reinterpret_cast<const u32x2*>(&sX[lds_off<RBX, true>(lcol, 32 * pb + 8 * q + 4 * g2)]);
      uint16_t* yr = y + (trow * H + h) * size_t(P) + 4 * g2;
#pragma unroll
      for (int pb = 0; pb < P / 32; ++pb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2 xv = xr[pb][q];
          const float xs[4] = {bf16_lo(xv[0]), bf16_hi(xv[0]), bf16_lo(xv[1]), bf16_hi(xv[1])};
          float o[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) o[rr] = acc[pb][4 * q + rr] + Dh * xs[rr];
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
                     const int4* tab, hipStream_t st, const StageEv& ev) {
  const int cps = kSC / s.Q;
  const int nsc = (s.nc + cps - 1) / cps;   // = ceil(T / 256) for equal-length rows
  const long blocks = long(s.b) * nsc * s.H;
  auto go = [&](auto kern) {
    hipExtLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(kThreads), 0, st, ev.start, ev.stop, 0,
                          static_cast<const uint16_t*>(x), CB, static_cast<const uint16_t*>(C), Acs, dtq, Hb, D,
                          static_cast<uint16_t*>(y), tab, s.T, s.H, s.G, s.Q, s.nc, nsc);
  };
  // one chunk per super-chunk: its H_c^T is staged in LDS
  if (s.Q == kSC)
    tab ? go(chunk_scan_mfma_kernel<N, P, true, true>) : go(chunk_scan_mfma_kernel<N, P, true, false>);
  else
    tab ? go(chunk_scan_mfma_kernel<N, P, false, true>) : go(chunk_scan_mfma_kernel<N, P, false, false>);
  return hipGetLastError();
}

template <int N>
hipError_t launch_n(const FwdShape& s, const void* x, const uint16_t* CB, const void* C,
                    const float* Acs, const float* dtq, const uint16_t* Hb, const float* D, void* y,
                    const int4* tab, hipStream_t st, const StageEv& ev) {
  switch (s.P) {
    case 32: return launch_np<N, 32>(s, x, CB, C, Acs, dtq, Hb, D, y, tab, st, ev);
    case 64: return launch_np<N, 64>(s, x, CB, C, Acs, dtq, Hb, D, y, tab, st, ev);
    case 128: return launch_np<N, 128>(s, x, CB, C, Acs, dtq, Hb, D, y, tab, st, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_scan_mfma(const FwdShape& s, const void* x, const uint16_t* CB,
                                  const void* C, const float* Acs, const float* dtq,
                                  const uint16_t* Hb, const float* D, void* y, const int4* tab,
                                  hipStream_t st, const StageEv& ev) {
  switch (s.N) {
    case 32: return launch_n<32>(s, x, CB, C, Acs, dtq, Hb, D, y, tab, st, ev);
    case 64: return launch_n<64>(s, x, CB, C, Acs, dtq, Hb, D, y, tab, st, ev);
    case 128: return launch_n<128>(s, x, CB, C, Acs, dtq, Hb, D, y, tab, st, ev);
    case 256: return launch_n<256>(s, x, CB, C, Acs, dtq, Hb, D, y, tab, st, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace ssd
