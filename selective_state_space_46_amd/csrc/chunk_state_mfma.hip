// chunk_state_mfma.hip -- chunk states on the bf16 matrix cores.
//
//   S_c^T[p][n] = sum_{s in chunk c} W[s][p] B_s[n],   W[s][p] = exp(Acs_{Q-1} - Acs_s) dt_s x_s[p]
//
// the per-chunk final-state block of the semiseparable form (youngju.dev
// "Mamba / selective SSM", "State Space Dualityの発見": h = sum_j abar_{T:j}
// bbar_j x_j^T with bbar_j = dt_j B_j), computed as the matrix product
// W^T (P x Q) . B (Q x N) contracted over the chunk's tokens
// ("SSDアルゴリズムとチャンク分割": inside a chunk, matrix products).
//
// The work-group first computes its chunk's in-chunk cumulative sums
// Acs_s = sum_{k <= s} dt_k A_h (the decay exponents; on this path it replaces
// chunk_cumsum.hip) and writes them, with dt, for state_passing and
// chunk_scan.
//
// Work-group: one (batch, chunk, head), 8 waves. The
// token axis is the contraction axis while x and B are stored token-major, so
// each 64-token slice is copied into LDS in its natural row-major order
// (coalesced 16-byte rows; W = w_s x_s scaled in fp32 per token row before its
// single bf16 rounding) and the MFMA operands are read transposed with
// ds_read_b64_tr_b16 (see mfma_util.h). The next slice's rows are loaded
// into registers while the current one feeds the matrix cores. Each wave owns
// (P/32)*(N/32)/8 output tiles of 32 x 32 (fp32 accumulators; one for
// headdim 64, dstate 128). One head per work-group and eight waves measured
// faster on MI355X than a head pair sharing the B slice (fewer accumulators,
// twice the work-groups) or four waves (half the loads in flight per CU).
// Output tiles go to HBM as fp32 rows of 32 consecutive n.
#include "mfma_util.h"

namespace ssd {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kSK = 64;          // tokens per contraction slice
constexpr int kMaxQ = 256;

// C B^T inside each chunk, once per B/C group (the same launch, work-groups
// placed before the chunk-state ones):
//   CB[l][s] = C_l . B_s      for l, s in the same chunk, s <= l (32 x 32 tiles)
// These are the dot products of the semiseparable matrix M_ij = C_i^T
// abar_{i:j} B_j before its decay (youngju.dev "Mamba / selective SSM",
// section "State Space Dualityの発見"); they depend only on B and C, which the
// heads of one group share (Qiita "Mamba-2" article, section 4.1: heads like
// multi-head attention, B/C per group). chunk_scan applies the per-head decay
// and causal mask to them.
//
// One wave per tile (batch, chunk, group, 32-row block l, 32-column block
// s <= l): the C_l and B_s rows load straight from memory (k = dstate; rows are
// dstate-contiguous) as one batch, N/16 MFMAs follow, and the tile is written
// as bf16 in MFMA result order: lane L holds rows 8(r/4) + 4(L/32) + r%4 of
// column L%32, exactly the B-operand fragments chunk_scan feeds to its next
// MFMA, loaded there with two coalesced 16-byte reads per lane.
// Layout: CB [b, nc, G, ntile, 64, 16] bf16 with ntile = lpc(lpc+1)/2,
// lpc = Q/32, tile (s, l) of a chunk at index l(l+1)/2 + s.
// BOTH (the backward's recomputation): the tiles stay fp32 (16 floats per
// lane, 4 KB per tile, at the same index), and the same products with the
// roles of the two operands swapped go to CBt, where lane L holds column
// s = L%32 and the registers run over rows l. The backward takes sums of
// these products that largely cancel, so they are not rounded to bf16.
template <int N, bool BOTH = false>
__device__ __forceinline__ void chunk_scores_tile(const uint16_t* __restrict__ Bm,
                                                  const uint16_t* __restrict__ Cm,
                                                  uint16_t* __restrict__ CB, uint16_t* __restrict__ CBt,
                                                  const int4* __restrict__ tab, int T, int G, int Q, int nc,
                                                  long wid, int lane) {
  const int lpc = Q / 32;
  const int ntile = lpc * (lpc + 1) / 2;
  const int l32 = lane & 31, g2 = lane >> 5;
  long rest = wid;
  const int ti = int(rest % ntile); rest /= ntile;
  const int g = int(rest % G); rest /= G;
  const int c = int(rest % nc);
  const int b = int(rest / nc);
  int i = 0;                                    // tile ti = i (i + 1) / 2 + j, j <= i
  while ((i + 1) * (i + 2) / 2 <= ti) ++i;
  const int j = ti - i * (i + 1) / 2;
  const ChunkRows cr0 = chunk_rows(tab, b, c, T, Q);
  if (32 * i >= cr0.n) return;                  // row block past the valid tokens: never read

  const int tl = 32 * i + l32, ts = 32 * j + l32;   // rows inside the chunk
  const uint16_t* cr = Cm + ((cr0.r0 + min(tl, cr0.n - 1)) * G + g) * size_t(N) + 8 * g2;
  const uint16_t* br = Bm + ((cr0.r0 + min(ts, cr0.n - 1)) * G + g) * size_t(N) + 8 * g2;
  u32x4 cf[N / 16], bf[N / 16];
#pragma unroll
  for (int ks = 0; ks < N / 16; ++ks) {
    cf[ks] = keep_or_zero(tl < cr0.n, load16(cr + 16 * ks));
    bf[ks] = keep_or_zero(ts < cr0.n, load16(br + 16 * ks));
  }
  const size_t at = (((size_t(b) * nc + c) * G + g) * ntile + ti) * 1024 + size_t(lane) * 16;
  auto store32 = [&](uint16_t* dstbase, const f32x16& acc) {
    f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(dstbase) + at);
#pragma unroll
    for (int m = 0; m < 4; ++m) dst[m] = f32x4{acc[4 * m], acc[4 * m + 1], acc[4 * m + 2], acc[4 * m + 3]};
  };
  auto store = [&](uint16_t* dstbase, const f32x16& acc) {
    u32x4 lo, hi;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      lo[m] = pack_bf16x2(acc[2 * m], acc[2 * m + 1]);
      hi[m] = pack_bf16x2(acc[8 + 2 * m], acc[8 + 2 * m + 1]);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(dstbase + at);
    dst[0] = lo;
    dst[1] = hi;
  };
  f32x16 acc = zero16();
#pragma unroll
  for (int ks = 0; ks < N / 16; ++ks) acc = mfma32x32x16(bf[ks], cf[ks], acc);   // rows s, column l
  if constexpr (BOTH) {
    store32(CB, acc);
    f32x16 acct = zero16();
#pragma unroll
    for (int ks = 0; ks < N / 16; ++ks) acct = mfma32x32x16(cf[ks], bf[ks], acct);   // rows l, column s
    store32(CBt, acct);
  } else {
    store(CB, acc);
  }
}

// MODE 0: the forward launch described above. MODE 1: the same, with the C B^T
// tiles also in the transposed orientation (CBt; the backward's
// recomputation of the forward). MODE 2 (backward): the state gradient each
// chunk contributes,
//   dS_c^T[p][n] = sum_{l in chunk c} exp(Acs_l) dy_l[p] C_l[n],
// the same product with x -> dy, B -> C and the per-token weight exp(Acs_l)
// (the chunk's inclusive cumulative decay up to l): no score tiles, and Acs /
// dt, recomputed here as in the forward, are not written again.
template <int N, int P, int MODE>
__global__ __launch_bounds__(kThreads) void chunk_state_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ dt,
    const float* __restrict__ A, float* __restrict__ Acs, float* __restrict__ dtq, float* __restrict__ S,
    const uint16_t* __restrict__ Cm, uint16_t* __restrict__ CB, uint16_t* __restrict__ CBt,
    const int4* __restrict__ tab, int T, int H, int G, int Q, int nc, int nscore_wg, long ntiles) {
  // the first nscore_wg work-groups compute C B^T tiles, one per wave
  if (int(blockIdx.x) < nscore_wg) {
    const long wid = long(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (wid < ntiles) chunk_scores_tile<N, MODE == 1>(Bm, Cm, CB, CBt, tab, T, G, Q, nc, wid, threadIdx.x & 63);
    return;                                     // no barrier on this path
  }
  constexpr int RBB = N / 8, RBW = P / 8;            // 16-byte chunks per row
  constexpr int CB_ = kSK * RBB, CW = kSK * RBW;     // chunks per slice
  constexpr int PER = (CB_ + CW + kThreads - 1) / kThreads;  // chunks per thread
  __shared__ __attribute__((aligned(16))) uint16_t sB[kSK * N];
  __shared__ __attribute__((aligned(16))) uint16_t sW[kSK * P];
  __shared__ float sw[kMaxQ];
  __shared__ float sacs[kMaxQ], sdt[kMaxQ], sred[kWaves];

  constexpr int NT = N / 32, PT = P / 32;
  constexpr int TILES = PT * NT;
  constexpr int TPW = (TILES + kWaves - 1) / kWaves;
  const int id = xcd_swizzle(int(blockIdx.x) - nscore_wg, int(gridDim.x) - nscore_wg);
  const int h = id % H;
  const int bc = id / H;
  const int c = bc % nc, b = bc / nc;
  const int g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_id();  // wave-uniform (scalar register)
  const int g2 = lane >> 5;
  const ChunkRows rows = chunk_rows(tab, b, c, T, Q);
  if (rows.n <= 0) return;                      // unused table slot: uniform, before any barrier

  // Acs_s = sum_{k <= s} dt_k A_h inside the chunk (dt = 0 past the end of
  // the sequence): one token per thread, a wave scan, then the totals of the
  // waves before. Written out for state_passing and chunk_scan.
  static_assert(kMaxQ <= kThreads, "one token per thread");
  const size_t arow = ((size_t(b) * H + h) * nc + c) * Q;
  {
    const float Ah = A[h];
    float d = 0.f;
    if (tid < rows.n) d = bf16_to_f32(dt[(rows.r0 + tid) * H + h]);
    float v = d * Ah;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(v, off, 64);
      if (lane >= off) v += o;
    }
    if (lane == 63) sred[wave] = v;
    __syncthreads();
    for (int w = 0; w < wave; ++w) v += sred[w];
    if (tid < Q) {
      if constexpr (MODE != 2) {
        Acs[arow + tid] = v;
        dtq[arow + tid] = d;
      }
      sacs[tid] = v;
      sdt[tid] = d;
    }
    __syncthreads();
  }
  // w_s = exp(Acs_{Q-1} - Acs_s) * dt_s for the whole chunk (MODE 2: exp(Acs_s))
  for (int i = tid; i < Q; i += kThreads)
    sw[i] = MODE == 2 ? exp_fast(sacs[i]) : exp_fast(sacs[Q - 1] - sacs[i]) * sdt[i];

  // this thread's 16-byte chunks of a slice: B rows first, then x rows
  auto load_slice = [&](int s0, u32x4 (&v)[PER]) {
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int e = tid + m * kThreads;
      if (e < CB_) {
        const int r = e / RBB, cc = e % RBB;
        const long row = rows.r0 + min(s0 + r, rows.n - 1);
        v[m] = load16(Bm + (row * G + g) * size_t(N) + 8 * cc);
      } else if (e < CB_ + CW) {
        const int r = (e - CB_) / RBW, cc = (e - CB_) % RBW;
        const long row = rows.r0 + min(s0 + r, rows.n - 1);
        v[m] = load16(x + (row * H + h) * size_t(P) + 8 * cc);
      }
    }
  };
  // rows past the chunk or the sequence become zeros; x rows are scaled by w_s
  auto store_slice = [&](int s0, const u32x4 (&v)[PER]) {
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int e = tid + m * kThreads;
      if (e < CB_) {
        const int r = e / RBB, cc = e % RBB;
        const bool in = s0 + r < rows.n;           // rows.n <= Q
        *reinterpret_cast<u32x4*>(&sB[lds_off<RBB>(r, 8 * cc)]) = keep_or_zero(in, v[m]);
      } else if (e < CB_ + CW) {
        const int r = (e - CB_) / RBW, cc = (e - CB_) % RBW;
        const float w = s0 + r < rows.n ? sw[s0 + r] : 0.f;
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(bf16_lo(v[m][q]) * w, bf16_hi(v[m][q]) * w);
        *reinterpret_cast<u32x4*>(&sW[lds_off<RBW>(r, 8 * cc)]) = o;
      }
    }
  };

  f32x16 acc[TPW];
#pragma unroll
  for (int m = 0; m < TPW; ++m) acc[m] = zero16();

  u32x4 pre[PER];
  load_slice(0, pre);
  for (int s0 = 0; s0 < Q; s0 += kSK) {
    __syncthreads();  // sw written / previous slice consumed
    store_slice(s0, pre);
    if (s0 + kSK < Q) load_slice(s0 + kSK, pre);
    __syncthreads();
    const int ksteps = min(kSK, Q - s0) / 16;
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int tile = wave + kWaves * m;
      if (tile < TILES) {
        const int pb = tile / NT, nb = tile % NT;
        for (int kk = 0; kk < ksteps; ++kk) {
          const int kb = 16 * kk + 8 * g2;
          const u32x4 a = frag_tr<RBW>(sW, kb, kb + 4, 32 * pb, lane);
          const u32x4 bb = frag_tr<RBB>(sB, kb, kb + 4, 32 * nb, lane);
          acc[m] = mfma32x32x16(a, bb, acc[m]);
        }
      }
    }
  }

  const int l32 = lane & 31;
  float* out = S + ((size_t(b) * nc + c) * H + h) * size_t(P) * N;
#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int tile = wave + kWaves * m;
    if (tile < TILES) {
      const int pb = tile / NT, nb = tile % NT;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int p = 32 * pb + 8 * (q / 4) + 4 * g2 + (q % 4);
        out[size_t(p) * N + 32 * nb + l32] = acc[m][q];
      }
    }
  }
}

template <int N, int P, int MODE>
hipError_t launch_np(const FwdShape& s, const void* x, const void* B, const void* C, const void* dt,
                     const float* A, float* Acs, float* dtq, float* S, uint16_t* CB, uint16_t* CBt, const int4* tab,
                     hipStream_t st, const StageEv& ev) {
  const int lpc = s.Q / 32;
  const long ntiles = MODE == 2 ? 0 : long(s.b) * s.nc * s.G * (lpc * (lpc + 1) / 2);
  // score work-groups first (they start with the first wave of work-groups),
  // padded to a multiple of 8 so the chunk-state work-groups keep their XCD
  const long nscore = ((ntiles + kWaves - 1) / kWaves + 7) / 8 * 8;
  const long blocks = nscore + long(s.b) * s.nc * s.H;
  hipExtLaunchKernelGGL((chunk_state_mfma_kernel<N, P, MODE>), dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                        ev.start, ev.stop, 0, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(B),
                        static_cast<const uint16_t*>(dt), A, Acs, dtq, S, static_cast<const uint16_t*>(C), CB,
                        CBt, tab, s.T, s.H, s.G, s.Q, s.nc, int(nscore), ntiles);
  return hipGetLastError();
}

template <int N, int MODE>
hipError_t launch_n(const FwdShape& s, const void* x, const void* B, const void* C, const void* dt,
                    const float* A, float* Acs, float* dtq, float* S, uint16_t* CB, uint16_t* CBt, const int4* tab,
                    hipStream_t st, const StageEv& ev) {
  switch (s.P) {
    case 32: return launch_np<N, 32, MODE>(s, x, B, C, dt, A, Acs, dtq, S, CB, CBt, tab, st, ev);
    case 64: return launch_np<N, 64, MODE>(s, x, B, C, dt, A, Acs, dtq, S, CB, CBt, tab, st, ev);
    case 128: return launch_np<N, 128, MODE>(s, x, B, C, dt, A, Acs, dtq, S, CB, CBt, tab, st, ev);
  }
  return hipErrorInvalidValue;
}

template <int MODE>
hipError_t launch_mode(const FwdShape& s, const void* x, const void* B, const void* C, const void* dt,
                       const float* A, float* Acs, float* dtq, float* S, uint16_t* CB, uint16_t* CBt,
                       const int4* tab, hipStream_t st, const StageEv& ev) {
  switch (s.N) {
    case 32: return launch_n<32, MODE>(s, x, B, C, dt, A, Acs, dtq, S, CB, CBt, tab, st, ev);
    case 64: return launch_n<64, MODE>(s, x, B, C, dt, A, Acs, dtq, S, CB, CBt, tab, st, ev);
    case 128: return launch_n<128, MODE>(s, x, B, C, dt, A, Acs, dtq, S, CB, CBt, tab, st, ev);
    case 256: return launch_n<256, MODE>(s, x, B, C, dt, A, Acs, dtq, S, CB, CBt, tab, st, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_state_mfma(const FwdShape& s, const void* x, const void* B, const void* C,
                                   const void* dt, const float* A, float* Acs, float* dtq,
                                   float* S, uint16_t* CB, const int4* tab, hipStream_t st,
                                   const StageEv& ev) {
  return launch_mode<0>(s, x, B, C, dt, A, Acs, dtq, S, CB, nullptr, tab, st, ev);
}

hipError_t launch_chunk_state_mfma_bwd(const FwdShape& s, const void* x, const void* B, const void* C,
                                       const void* dt, const float* A, float* Acs, float* dtq, float* S,
                                       uint16_t* CB, uint16_t* CBt, hipStream_t st) {
  return launch_mode<1>(s, x, B, C, dt, A, Acs, dtq, S, CB, CBt, nullptr, st, StageEv{});
}

hipError_t launch_chunk_dstates_mfma(const FwdShape& s, const void* dy, const void* C, const void* dt,
                                     const float* A, float* dS, hipStream_t st) {
  return launch_mode<2>(s, dy, C, nullptr, dt, A, nullptr, nullptr, dS, nullptr, nullptr, nullptr, st, StageEv{});
}

}  // namespace ssd
