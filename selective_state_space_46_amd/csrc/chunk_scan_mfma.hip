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
// head; W waves. The C B^T tiles come precomputed once per group (by the
// chunk_state launch, chunk_state_mfma.hip) in MFMA-fragment order. The
// super-chunk is cut into eight 32-row blocks l; with W = 4 wave w owns
// blocks w and 7-w so that the causal triangle splits evenly, with W = 8 one
// block each (twice the waves on the same LDS, for latency hiding): wave w <
// 4 block w, wave w >= 4 block 11 - w, so the two waves that share a SIMD
// (w and w + 4) hold blocks k and 7 - k, 9 tiles on every SIMD. The output is produced transposed (y^T: rows p, lane = token
// l), which makes every per-token factor one multiplier per lane:
//   1. y^T = H_c^T C_l^T (k = dstate): H_c staged once in LDS as stored (bf16,
//      fragment order, from the fused walk or state_passing, see hb_off) when
//      the super-chunk is one chunk, C_l rows from the copy of C that the
//      tiles' producer leaves in operand order (1 KB contiguous per load;
//      from C itself each load would read 32 bytes in each of 32 rows); then
//      y^T *= exp(Acs_l).
//   2. for each column block s <= l of the chunk: the C B^T tile (lane =
//      column l, registers = rows s in runs of 4) times the decay, rounded to
//      bf16, is the B operand of y^T += X^T G^T under a k permutation that the
//      X operand reproduces: x sits in LDS in natural token-major order
//      (swizzled 16-byte chunks) and is read transposed with
//      ds_read_b64_tr_b16. With W = 8 a block's tiles all load at once; with
//      W = 4 through a ring of three buffers, two tiles ahead of use.
//   3. + D x (x from the same LDS tile), bf16 rounding, 8-byte stores of 4
//      consecutive p; where the super-chunk is one chunk the rounded rows go
//      back through the x tile (after a barrier: no wave reads x any more) and
//      leave as 16-byte pieces of whole token rows.
// SEG (rows cut into segments by the fused chunk-state walk): Hb holds the
// local states, from zero at each segment's start; the state entering chunk
// c of segment k >= 1 is Hb_c + exp(cdec_c) Hin_k (Hin fp32 [b, nseg, H,
// P * N] in the same fragment order, the state entering each segment;
// cdec_c <= 0), formed in fp32 where
// H_c is staged or loaded and rounded to bf16 once. Where exp(cdec_c)
// underflows to zero (a decayed segment start) the correction is exactly
// zero and Hin is not read. Packed sequences (VARLEN with SEG): the row of
// chunk slots is cut into segments the same way; the walk leaves cdec = -inf
// on every chunk after a sequence begins inside its segment, so only the
// chunks of the sequence the segment continues take a correction.
#include "mfma_util.h"

namespace ssd {
namespace {

constexpr int kSC = 256;          // tokens per super-chunk
constexpr float kLog2e = 1.4426950408889634f;

// 8 bf16 of a local state plus alpha times the 8 matching fp32 of Hin, rounded
// to bf16 once
__device__ __forceinline__ u32x4 seg_combine(const u32x4& v, const float* hin, float alpha) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(hin);
  const f32x4 b = *reinterpret_cast<const f32x4*>(hin + 4);
  return u32x4{pack_bf16x2(bf16_lo(v[0]) + alpha * a[0], bf16_hi(v[0]) + alpha * a[1]),
               pack_bf16x2(bf16_lo(v[1]) + alpha * a[2], bf16_hi(v[1]) + alpha * a[3]),
               pack_bf16x2(bf16_lo(v[2]) + alpha * b[0], bf16_hi(v[2]) + alpha * b[1]),
               pack_bf16x2(bf16_lo(v[3]) + alpha * b[2], bf16_hi(v[3]) + alpha * b[3])};
}

// VARLEN: chunk rows from the chunk table tab (packed sequences), else the
// equal-length layout (tab unused). SEG: the segment correction above.
template <int N, int P, bool HLDS, bool VARLEN, bool SEG, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(W == 8 && P <= 64 ? 4 : 1)))
void chunk_scan_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ CB, const uint16_t* __restrict__ Cf,
    const float* __restrict__ Acs, const float* __restrict__ dtq, const uint16_t* __restrict__ Hb,
    const float* __restrict__ D, uint16_t* __restrict__ y, const int4* __restrict__ tab, int T, int H,
    int G, int Q, int nc, int nsc, const float* __restrict__ Hin, const float* __restrict__ cdec, int nseg,
    int seglen) {
  constexpr int kThreads = 64 * W;
  constexpr int NB = 8 / W;   // 32-row blocks per wave
  constexpr int RBX = P / 8;  // 16-byte chunks per X' row
  __shared__ __attribute__((aligned(16))) uint16_t sX[kSC * P];
  // H_c staged as it is stored, in fragment order (hb_off)
  __shared__ __attribute__((aligned(16))) uint16_t sH[HLDS ? P * N : 8];
  __shared__ __attribute__((aligned(16))) float sA[kSC];  // Acs * log2(e)
  __shared__ __attribute__((aligned(16))) float sF[kSC];  // exp(Acs[block end] - Acs_s) * dt_s
  __shared__ __attribute__((aligned(16))) float sL[kSC];  // log2(dt_s) - Acs_s log2(e)

  // HLDS kernels run only with one chunk per super-chunk: Q as a constant
  // lets every index below fold
  if constexpr (HLDS) Q = kSC;
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
  // (one chunk per super-chunk: its table entry read once)
  const ChunkRows row_c0 = chunk_rows(VARLEN ? tab : static_cast<const int4*>(nullptr), b, c0, T, Q);
  auto crows = [&](int ci) {
    if constexpr (HLDS) return ci == 0 ? row_c0 : ChunkRows{0, 0};
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
  // SEG: the segment of chunk c and whether a state from before the segment
  // can enter it
  auto seg_of = [&](int c, int& k, bool& later) {
    k = min(c / seglen, nseg - 1);
    later = k > 0;
  };

  // C B^T tiles of 32-row block i: tile jj (column block jfirst + jj) of the
  // block's row of its chunk's lower triangle, this lane's 32 bytes
  auto tile_src = [&](int i) {
    const int jf = (i / lpc) * lpc, cgi = c0 + i / lpc, ir = i - jf;
    return reinterpret_cast<const u32x4*>(
        CB + (((size_t(b) * nc + cgi) * G + g) * ntile + size_t(ir) * (ir + 1) / 2) * 1024 +
        size_t(lane) * 16);
  };
  // a block's first loads: its diagonal tile (W = 4; with W = 8 it comes
  // with the other tiles, after the C rows are used), its first tile, its C
  // rows (k = dstate, rows clamped into the tensor; zeroed past the end at use)
  auto issue_block_loads = [&](int i, u32x4 (&td)[2], u32x4 (&tn)[2], u32x4 (&cfv)[N / 16]) {
    const u32x4* ts = tile_src(i);
    const int ir = i - (i / lpc) * lpc;
    if constexpr (W != 8) {
      td[0] = ts[ir * 128];
      td[1] = ts[ir * 128 + 1];
    }
    tn[0] = ts[0];
    tn[1] = ts[1];
    // C in operand order, written with the tiles (Cf, zeros past the
    // chunk's tokens): each load is 1 KB contiguous per wave
    const uint16_t* cr = Cf + ((((size_t(b) * nc + c0 + i / lpc) * G + g) * lpc + i % lpc) * (N / 16) * 64 + lane) * 8;
#pragma unroll
    for (int ks = 0; ks < N / 16; ++ks) cfv[ks] = load16(cr + 512 * ks);
  };
  // the wave's first block: with W = 8 (one block each) waves w and w + 4
  // share a SIMD, so wave w >= 4 takes block 11 - w: every SIMD then holds
  // blocks k and 7 - k, 9 tiles
  const int blk0 = (W == 8 && wave >= 4) ? 11 - wave : wave;

  // ---- staging: the per-token tables (Acs, the per-token factor), H_c and
  // x into LDS, and the first block's tiles and C rows into registers. Every
  // load is issued before the first value is used, tables first and the
  // register-only loads last: the vector memory counter retires loads in
  // issue order, so each wait below covers only what is needed there (a
  // wait for the tables or H would otherwise also wait for the C rows).
  // tables: one token per thread (kSC <= threads)
  static_assert(kSC <= kThreads, "one table entry per thread");
  // (loads unconditional, at an in-bounds index, and masked where used, so
  // that nothing waits for them before the loads below are issued)
  const int tq = min(tid, kSC - 1);
  const bool tvalid = tid < kSC && crows(tq / Q).n > 0;
  float ta, tl, td;
  {
    const size_t row = ((size_t(b) * H + h) * nc + min(c0 + tq / Q, nc - 1)) * Q;
    const int q = tq % Q;
    ta = Acs[row + q];
    tl = Acs[row + (q | 31)];
    td = dtq[row + q];
  }
  // H_c in fragment order (hb_off), copied as it is (with segments, plus
  // alpha times the state entering the segment, stored in the same order)
  constexpr int kPieces = HLDS ? P * N / 8 : 1;      // 16-byte pieces of one state
  constexpr int KP = (kPieces + kThreads - 1) / kThreads;
  u32x4 hv[KP];
  float alpha = 0.f;                                 // uniform
  int sgk = 0;                                       // the chunk's segment (uniform)
  if constexpr (HLDS) {
    const uint16_t* hsrc = Hb + ((size_t(b) * nc + c0) * H + h) * size_t(P) * N;
    bool later = false;
    if constexpr (SEG) seg_of(c0, sgk, later);
    // the weight of the state entering the segment (where it underflows to
    // zero the correction adds exactly zero and is skipped)
    if (SEG && later) alpha = exp_fast(cdec[(size_t(b) * H + h) * nc + c0]);
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int e = min(tid + k * kThreads, kPieces - 1);
      hv[k] = load16(hsrc + 8 * size_t(e));
    }
  }
  // raw x, token-major, swizzled. Thread tid copies 16-byte chunk tid % RBX
  // of rows tid / RBX + k kStep; kStep is a multiple of the swizzle period
  // (16 rows), so every row of the thread has the same swizzle and its LDS
  // offsets differ by constants.
  static_assert(kThreads % RBX == 0 && (kThreads / RBX) % 16 == 0, "x staging shape");
  constexpr int kStep = kThreads / RBX;
  const int xr0 = tid / RBX, xcc = tid % RBX;
  u32x4 xv[kSC / kStep];
  bool xok[kSC / kStep];       // rows past their chunk's tokens: zeros, applied when written
  if (fast) {
    const uint16_t* src = x + ((rows0.r0 + xr0) * H + h) * size_t(P) + 8 * xcc;
    const size_t step = size_t(kStep) * H * P;
#pragma unroll
    for (int k = 0; k < kSC / kStep; ++k) {
      xv[k] = load16(src + k * step);
      xok[k] = opaque(1) != 0;   // not a constant: the mask stays at the writes below
    }
  } else {
#pragma unroll
    for (int k = 0; k < kSC / kStep; ++k) {
      const int r = xr0 + k * kStep;
      const ChunkRows cr = crows(r / Q);
      const int rq = r % Q;
      // a chunk with no valid rows (past the last chunk, or an unused table
      // slot) reads a valid row of another chunk instead: any in-bounds row
      const long row = cr.n > 0 ? cr.r0 + min(rq, cr.n - 1) : rowsv.r0;
      xv[k] = load16(x + (row * H + h) * size_t(P) + 8 * xcc);
      xok[k] = rq < cr.n;
    }
  }
  u32x4 pre_tdiag[2], pre_tnext[2], pre_cf[N / 16];
  if ((blk0 % lpc) * 32 < crows(blk0 / lpc).n) issue_block_loads(blk0, pre_tdiag, pre_tnext, pre_cf);

  if (tid < kSC) {
    const float a = tvalid ? ta * kLog2e : 0.f, d = tvalid ? td : 0.f;
    sA[tid] = a;
    sF[tid] = tvalid ? __builtin_amdgcn_exp2f(tl * kLog2e - a) * d : 0.f;  // exponent <= 0
    sL[tid] = __builtin_amdgcn_logf(d) - a;                               // log2; -inf where dt = 0
  }
  if constexpr (HLDS) {
    if (SEG && alpha != 0.f) {
      const float* hin = Hin + ((size_t(b) * nseg + sgk) * H + h) * size_t(P) * N;
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        const int e = min(tid + k * kThreads, kPieces - 1);
        hv[k] = seg_combine(hv[k], hin + 8 * size_t(e), alpha);   // Hin: the same order
      }
    }
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int e = tid + k * kThreads;
      if (kPieces % kThreads == 0 || e < kPieces) *reinterpret_cast<u32x4*>(&sH[8 * e]) = hv[k];
    }
  }
  {
    uint16_t* dst = &sX[lds_off<RBX, true>(xr0, 8 * xcc)];
#pragma unroll
    for (int k = 0; k < kSC / kStep; ++k) *reinterpret_cast<u32x4*>(dst + k * kStep * P) = keep_or_zero(xok[k], xv[k]);
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
  // YLDS (one chunk per super-chunk): the rounded outputs of the wave's
  // blocks wait in registers (yv[1] the last block's, yv[0] the first's when
  // a wave has two) until every wave has finished its tiles, then go through
  // this wave's own rows of the x tile (no wave reads x any more) so that
  // each store instruction writes whole 16-byte pieces of consecutive token
  // rows; stored straight from the accumulators, each instruction would
  // write 16 bytes in each of 32 token rows.
  constexpr bool YLDS = HLDS;
  u32x2 yv[2][P / 32][4];
  int yblk[2] = {-1, -1};          // the blocks whose outputs yv holds (uniform), -1: none
  for (int which = 0; which < NB; ++which) {
    const int i = which ? 7 - wave : blk0;  // 32-row block of the super-chunk
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
      for (int m = 0; m < 2; ++m) {
        if constexpr (W != 8) tdiag[m] = pre_tdiag[m];
        tnext[m] = pre_tnext[m];
      }
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
    const int hlane = 256 * g2 + 4 * l32;   // this lane's part of a fragment-order offset
    // segments, per-fragment path: this block's chunk's segment and the
    // weight of the state entering it (uniform)
    int sgb = 0;
    bool later_b = false;
    if constexpr (SEG && !HLDS) seg_of(cg, sgb, later_b);
    const float alpha_b = SEG && !HLDS && later_b ? exp_fast(cdec[(size_t(b) * H + h) * nc + cg]) : 0.f;
#pragma unroll
    for (int pb = 0; pb < P / 32; ++pb) {
      acc[pb] = zero16();
#pragma unroll
      for (int ks = 0; ks < N / 16; ++ks) {
        u32x4 hf;
        // eight consecutive n of row p: two runs of four in fragment order
        // (in LDS: the 32 lanes of each half read 256 contiguous bytes per run).
        // With n = 16 ks + 8 g2, hb_off(p, n) = hlane + 256 ((pb N / 32 + ks / 2) 4
        // + 2 (ks % 2)) with the per-lane part hlane = 256 g2 + 4 l32, and the
        // run of n + 4 sits 128 elements (32 runs) after it
        const int p = 32 * pb + l32, n = 16 * ks + 8 * g2;
        if constexpr (HLDS) {
          const int o = hlane + 256 * ((pb * (N / 32) + ks / 2) * 4 + 2 * (ks % 2));
          const u32x2 lo = *reinterpret_cast<const u32x2*>(&sH[o]);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(&sH[o + 128]);
          hf = u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
          const uint16_t* hs = Hb + ((size_t(b) * nc + cg) * H + h) * size_t(P) * N;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(hs + hb_off(p, n, N));
          const u32x2 hi = *reinterpret_cast<const u32x2*>(hs + hb_off(p, n + 4, N));
          hf = u32x4{lo[0], lo[1], hi[0], hi[1]};
          if (SEG && alpha_b != 0.f) {
            const float* hin = Hin + ((size_t(b) * nseg + sgb) * H + h) * size_t(P) * N;
            const f32x4 a = *reinterpret_cast<const f32x4*>(hin + hb_off(p, n, N));
            const f32x4 c = *reinterpret_cast<const f32x4*>(hin + hb_off(p, n + 4, N));
            hf = u32x4{pack_bf16x2(bf16_lo(hf[0]) + alpha_b * a[0], bf16_hi(hf[0]) + alpha_b * a[1]),
                       pack_bf16x2(bf16_lo(hf[1]) + alpha_b * a[2], bf16_hi(hf[1]) + alpha_b * a[3]),
                       pack_bf16x2(bf16_lo(hf[2]) + alpha_b * c[0], bf16_hi(hf[2]) + alpha_b * c[1]),
                       pack_bf16x2(bf16_lo(hf[3]) + alpha_b * c[2], bf16_hi(hf[3]) + alpha_b * c[3])};
          }
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
    if constexpr (W == 8) {
      // one block per wave (at most 7 off-diagonal tiles): all of them and
      // the diagonal one in flight at once, in the registers the C rows held
      // until here
      u32x4 tall[7][2], tdg[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) tall[0][u] = tnext[u];
#pragma unroll
      for (int t = 1; t < 7; ++t)
        if (t < irel) load_tile(t, tall[t]);
      load_tile(irel, tdg);
#pragma unroll
      for (int t = 0; t < 7; ++t)
        if (t < irel) apply(t, tall[t], false);
      apply(irel, tdg, true);
    } else {
      // off-diagonal tiles through a ring of three buffers: the next two
      // tiles load while one is applied (no register copies)
      u32x4 tB[2], tC[2];
      if (1 < irel) load_tile(1, tB);
      if (2 < irel) load_tile(2, tC);
#pragma unroll 1
      for (int jj = 0; jj < irel; jj += 3) {
        apply(jj, tnext, false);
        if (jj + 3 < irel) load_tile(jj + 3, tnext);
        if (jj + 1 < irel) {
          apply(jj + 1, tB, false);
          if (jj + 4 < irel) load_tile(jj + 4, tB);
        }
        if (jj + 2 < irel) {
          apply(jj + 2, tC, false);
          if (jj + 5 < irel) load_tile(jj + 5, tC);
        }
      }
      apply(irel, tdiag, true);
    }

    // ---- epilogue: + D x (x from the LDS tile), round; store 4 consecutive p
    // (8 bytes) per run, or keep them for the row-wise store below
    if constexpr (YLDS) {
      u32x2 cur[P / 32][4];
#pragma unroll
      for (int pb = 0; pb < P / 32; ++pb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2 xv = *reinterpret_cast<const u32x2*>(&sX[lds_off<RBX, true>(lcol, 32 * pb + 8 * q + 4 * g2)]);
          const float xs[4] = {bf16_lo(xv[0]), bf16_hi(xv[0]), bf16_lo(xv[1]), bf16_hi(xv[1])};
          float o[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) o[rr] = acc[pb][4 * q + rr] + Dh * xs[rr];
          cur[pb][q] = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        }
      // slot 0: a first block of two (uniform branch)
      if (NB == 2 && which == 0) {
        yblk[0] = i;
#pragma unroll
        for (int pb = 0; pb < P / 32; ++pb)
#pragma unroll
          for (int q = 0; q < 4; ++q) yv[0][pb][q] = cur[pb][q];
      } else {
        yblk[1] = i;
#pragma unroll
        for (int pb = 0; pb < P / 32; ++pb)
#pragma unroll
          for (int q = 0; q < 4; ++q) yv[1][pb][q] = cur[pb][q];
      }
    } else if (tok_ok) {
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
  if constexpr (YLDS) {
    // every wave is done with x (tiles and D x): each overwrites its own
    // block's 32 rows of the x tile with its outputs, at the addresses its D x
    // reads came from, and reads them back as 16-byte row pieces (RBX lanes
    // per row, 64 / RBX rows per instruction) for the stores
    __syncthreads();
#pragma unroll
    for (int sl = 2 - NB; sl < 2; ++sl) {
      if (yblk[sl] < 0) continue;       // uniform
      const int i = yblk[sl];
      const ChunkRows cr = crows(i / lpc);
      const int rq0 = (i % lpc) * 32;
#pragma unroll
      for (int pb = 0; pb < P / 32; ++pb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<u32x2*>(&sX[lds_off<RBX, true>(32 * i + l32, 32 * pb + 8 * q + 4 * g2)]) = yv[sl][pb][q];
      constexpr int RPI = 64 / RBX;     // rows per store instruction
      const int cc = lane % RBX;
#pragma unroll
      for (int u = 0; u < 32 / RPI; ++u) {
        const int r = u * RPI + lane / RBX;   // row of the block
        const u32x4 v = *reinterpret_cast<const u32x4*>(&sX[lds_off<RBX, true>(32 * i + r, 8 * cc)]);
        if (rq0 + r < cr.n)
          *reinterpret_cast<u32x4*>(y + ((cr.r0 + rq0 + r) * H + h) * size_t(P) + 8 * cc) = v;
      }
    }
  }
}

template <int N, int P>
hipError_t launch_np(const FwdShape& s, const void* x, const uint16_t* CB, const uint16_t* Cf,
                     const float* Acs, const float* dtq, const uint16_t* Hb, const float* D, void* y,
                     const int4* tab, hipStream_t st, const StageEv& ev, const SegStates& sg) {
  const int cps = kSC / s.Q;
  const int nsc = (s.nc + cps - 1) / cps;   // = ceil(T / 256) for equal-length rows
  const long blocks = long(s.b) * nsc * s.H;
  // waves per work-group: 8 (one 32-row block each, 128 registers) where
  // dstate 256 and the staged H_c leave two 4-wave work-groups per unit with
  // 254 registers each; 4 elsewhere
  constexpr int W = N == 256 ? 8 : 4;
  auto go = [&](auto kern, int w) {
    hipExtLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(64 * w), 0, st, ev.start, ev.stop, 0,
                          static_cast<const uint16_t*>(x), CB, Cf, Acs, dtq, Hb, D,
                          static_cast<uint16_t*>(y), tab, s.T, s.H, s.G, s.Q, s.nc, nsc, sg.Hin, sg.cdec, sg.nseg,
                          sg.seglen);
  };
  const bool seg = sg.nseg > 1 || sg.var;
  if (!Cf || (seg && (!sg.Hin || !sg.cdec || sg.seglen < 1 || sg.var != (tab != nullptr))))
    return hipErrorInvalidValue;
  // packed sequences through segments: only where the fused walk runs
  if constexpr (N >= 128) {
    if (seg && tab) {
      if (s.Q == kSC) go(chunk_scan_mfma_kernel<N, P, true, true, true, W>, W);
      else go(chunk_scan_mfma_kernel<N, P, false, true, true, 4>, 4);
      return hipGetLastError();
    }
  } else {
    if (seg && tab) return hipErrorInvalidValue;
  }
  // one chunk per super-chunk: its H_c^T is staged in LDS
  if (s.Q == kSC) {
    if (seg) go(chunk_scan_mfma_kernel<N, P, true, false, true, W>, W);
    else if (tab) go(chunk_scan_mfma_kernel<N, P, true, true, false, W>, W);
    else go(chunk_scan_mfma_kernel<N, P, true, false, false, W>, W);
  } else {
    if (seg) go(chunk_scan_mfma_kernel<N, P, false, false, true, 4>, 4);
    else if (tab) go(chunk_scan_mfma_kernel<N, P, false, true, false, 4>, 4);
    else go(chunk_scan_mfma_kernel<N, P, false, false, false, 4>, 4);
  }
  return hipGetLastError();
}

template <int N>
hipError_t launch_n(const FwdShape& s, const void* x, const uint16_t* CB, const uint16_t* Cf,
                    const float* Acs, const float* dtq, const uint16_t* Hb, const float* D, void* y,
                    const int4* tab, hipStream_t st, const StageEv& ev, const SegStates& sg) {
  switch (s.P) {
    case 32: return launch_np<N, 32>(s, x, CB, Cf, Acs, dtq, Hb, D, y, tab, st, ev, sg);
    case 64: return launch_np<N, 64>(s, x, CB, Cf, Acs, dtq, Hb, D, y, tab, st, ev, sg);
    case 128: return launch_np<N, 128>(s, x, CB, Cf, Acs, dtq, Hb, D, y, tab, st, ev, sg);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_scan_mfma(const FwdShape& s, const void* x, const uint16_t* CB,
                                  const uint16_t* Cf, const float* Acs, const float* dtq,
                                  const uint16_t* Hb, const float* D, void* y, const int4* tab,
                                  hipStream_t st, const StageEv& ev, const SegStates& sg) {
  switch (s.N) {
    case 32: return launch_n<32>(s, x, CB, Cf, Acs, dtq, Hb, D, y, tab, st, ev, sg);
    case 64: return launch_n<64>(s, x, CB, Cf, Acs, dtq, Hb, D, y, tab, st, ev, sg);
    case 128: return launch_n<128>(s, x, CB, Cf, Acs, dtq, Hb, D, y, tab, st, ev, sg);
    case 256: return launch_n<256>(s, x, CB, Cf, Acs, dtq, Hb, D, y, tab, st, ev, sg);
  }
  return hipErrorInvalidValue;
}

}  // namespace ssd
