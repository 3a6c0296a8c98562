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

// ---------------------------------------------------------------------------
// Chunk states and the passing between chunks in one pass (equal-length rows):
//
//   H_0 = init (or 0);  for c = 0 .. nc-1:  Hb_c = bf16(H_c),
//                       H_{c+1} = exp(Acs_c[Q-1]) H_c + S_c;   final = H_nc
//
// the recurrence of state_passing.hip folded into the chunk-state product
// (youngju.dev "Mamba / selective SSM", "SSDアルゴリズムとチャンク分割": the
// state handed from chunk to chunk; Qiita "Mamba-2" article, section 4.2,
// steps 2 and 3). A work-group owns one (batch row, head, 32 columns p of the
// head) and walks that row's chunks in order, its running state held in the
// fp32 accumulators of the matrix cores: at a chunk's start the accumulators
// (= H_c) go out as bf16 for chunk_scan, are scaled by the chunk's decay, and
// the chunk's products then accumulate on top, leaving H_{c+1}. The fp32 chunk
// states S_c never reach HBM (the two-kernel form writes and re-reads them).
//
// Tokens stream through 64-row slices of B (all of dstate) and x (the 32
// columns), copied straight from global memory into LDS (global_load_lds,
// 16 bytes per lane) in their natural swizzled row-major layout, three slices
// resident: one read while the next two load. The copies use no registers, so
// two slices stay in flight behind the one being multiplied. The MFMA
// operands are read transposed (ds_read_b64_tr_b16); the x fragment is scaled
// by w_s = exp(Acs_{Q-1} - Acs_s) dt_s there and rounded to bf16 once (the
// same W = w x as chunk_state_mfma_kernel). The product is taken as S[n][p]
// (rows n, lanes p), so a lane holds four consecutive n of one p: H_c leaves
// as runs of its [p][n] rows, init and final ([n][p]) as whole rows of p.
//
// Four compute waves issue only the slice copies; a fifth wave does every
// global store (H_c through LDS, the chunk's Acs / dt rows) and loads the dt
// rows two chunks ahead. The vector memory counter counts loads and stores
// together and the two may complete out of order, so a wave with both in
// flight waits for all of them at its next wait; the compute waves wait only
// for their own copies, by count. The two kinds of wave run separate loops
// that pass the same barriers.
// ---------------------------------------------------------------------------
constexpr int kChainWaves = 8;      // 4 compute waves + 4 store waves
constexpr int kChainThreads = 64 * kChainWaves;
constexpr int kChainCT = 256;        // compute threads (waves 0..3)
constexpr int kChainSK = 64;         // tokens per slice
constexpr int kChainStages = 3;      // slices resident in LDS

// vmcnt(n), the other counters left alone (low four bits of n in bits 3..0,
// high two in bits 15..14)
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Work-group barrier for LDS traffic only (the waves of this launch share
// nothing else through memory): this wave's LDS operations complete, then
// the barrier; the memory clobber keeps the compiler from moving memory
// accesses across it. Unlike __syncthreads it does not make each wave wait
// for its slice copies still in flight, which the copy protocol waits for
// by count instead.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One wave's direct copy of 64 x 16 bytes from global memory into LDS: lane
// L's 16 bytes land at dst + 16 L (dst wave-uniform; checked on MI355X).
__device__ __forceinline__ void copy_to_lds16(const uint16_t* src, uint16_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(dst), 16, 0, 0);
}

template <int N, int P, int SPC>
__global__ __launch_bounds__(kChainThreads) void chunk_state_chain_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ dt,
    const float* __restrict__ A, float* __restrict__ Acs, float* __restrict__ dtq, uint16_t* __restrict__ Hb,
    const float* __restrict__ init, float* __restrict__ fin, const uint16_t* __restrict__ Cm,
    uint16_t* __restrict__ CB, int T, int H, int G, int Q, int nc, int nchain, long ntiles) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_id();  // wave-uniform (scalar register)
  // work-groups past the chains compute C B^T tiles, one per wave
  if (int(blockIdx.x) >= nchain) {
    const long wid = long(int(blockIdx.x) - nchain) * kChainWaves + wave;
    if (wid < ntiles) chunk_scores_tile<N, false>(Bm, Cm, CB, nullptr, nullptr, T, G, Q, nc, wid, lane);
    return;                                     // no barrier on this path
  }
  constexpr int PB = 32, NPB = P / PB;
  constexpr int RBB = N / 8, RBX = PB / 8;      // 16-byte chunks per B row / x row slice
  constexpr int NCB = kChainSK * RBB / 64;      // wave copies per B slice
  static_assert(NCB % 4 == 0 && kChainSK * RBX == 256, "slice shape");
  constexpr int OPS = NCB / 4 + 1;              // copies per compute wave and slice
  constexpr int TPW = N / 128;                  // 32 x 32 tiles per compute wave
  constexpr int kHS = N + 8;                    // sH row stride (bf16): aligned 16-byte rows, 2-way writes
  constexpr int kDtL = kMaxQ / 64;              // dt values per store-wave lane and chunk
  // one array per slot: distinct LDS objects let the compiler see that reads
  // of one slot do not alias copies in flight into another
  __shared__ __attribute__((aligned(16))) uint16_t sB0[kChainSK * N], sB1[kChainSK * N], sB2[kChainSK * N];
  __shared__ __attribute__((aligned(16))) uint16_t sX0[kChainSK * PB], sX1[kChainSK * PB], sX2[kChainSK * PB];
  auto slotB = [&](int s) { return s == 0 ? sB0 : s == 1 ? sB1 : sB2; };
  auto slotX = [&](int s) { return s == 0 ? sX0 : s == 1 ? sX1 : sX2; };
  __shared__ __attribute__((aligned(16))) uint16_t sH[PB * kHS];
  __shared__ __attribute__((aligned(16))) float sacs[kMaxQ], sdt[kMaxQ], sw[kMaxQ];
  __shared__ float sdtq[2][kMaxQ], sred[4];

  const int id = xcd_swizzle(int(blockIdx.x), nchain);
  const int pb = id % NPB;
  const int bh = id / NPB;                      // b * H + h
  const int h = bh % H, b = bh / H;
  const int g = h / (H / G);
  const int l32 = lane & 31, g2 = lane >> 5;
  const int nsl = nc * SPC;                     // slices of the row
  const size_t hstate = size_t(P) * N;          // elements of one (b, h) state

  if (wave >= 4) {
    // ---- store waves: dt of chunks 0 and 1 first (store wave 0), then the
    // same barriers as the compute waves, in the same order. Four of them
    // (rather than one) keep the work-group a whole number of waves per SIMD,
    // which lets two work-groups share a compute unit.
    const int sv = wave - 4;
    // dt of chunk c, token lane + 64 i (0 past the row)
    auto dt_load = [&](int c, float (&v)[kDtL]) {
      const ChunkRows cr = chunk_rows(nullptr, b, c, T, Q);
#pragma unroll
      for (int i = 0; i < kDtL; ++i) {
        const int t = lane + 64 * i;
        const float raw = bf16_to_f32(dt[(cr.r0 + min(t, cr.n - 1)) * H + h]);
        v[i] = t < cr.n ? raw : 0.f;
      }
    };
    auto dt_put = [&](int slot, const float (&v)[kDtL]) {
#pragma unroll
      for (int i = 0; i < kDtL; ++i)
        if (lane + 64 * i < Q) sdtq[slot][lane + 64 * i] = v[i];
    };
    float pend[kDtL];
    if (sv == 0) {
      dt_load(0, pend);
      dt_put(0, pend);
      if (nc > 1) {
        dt_load(1, pend);
        dt_put(1, pend);
      }
    }
    lds_barrier();                            // [0]
    const int nsteps = (nsl + 2) / 3 * 3;
    for (int k = 0; k < nsteps; ++k) {
      lds_barrier();                            // [4] slice k in LDS
      if (k < nsl && k % SPC == 0) {
        const int c = k / SPC;
        if (sv == 0 && c >= 1 && c + 1 < nc) dt_put((c + 1) & 1, pend);   // loaded during chunk c - 1
        lds_barrier();                          // [1]
        if (sv == 0 && c + 2 < nc) dt_load(c + 2, pend);
        lds_barrier();                          // [2] sacs, sdt = chunk c
        const int t = 64 * sv + lane;
        if (pb == 0 && t < Q) {
          const size_t arow = (size_t(bh) * nc + c) * Q;
          Acs[arow + t] = sacs[t];
          dtq[arow + t] = sdt[t];
        }
        lds_barrier();                          // [3] sH = H_c
        // rows 8 sv .. 8 sv + 7 of H_c, and tokens 64 sv .. 64 sv + 63 of
        // the chunk's Acs / dt rows
        uint16_t* hdst = Hb + ((size_t(b) * nc + c) * H + h) * hstate + size_t(PB) * pb * N;
#pragma unroll
        for (int i = 0; i < PB / 4 * RBB / 64; ++i) {
          const int e = lane + 64 * i, pr = PB / 4 * sv + e / RBB, cc = e % RBB;
          *reinterpret_cast<u32x4*>(hdst + size_t(pr) * N + 8 * cc) =
              *reinterpret_cast<const u32x4*>(&sH[pr * kHS + 8 * cc]);
        }
      }
    }
    lds_barrier();                              // [5]
    lds_barrier();                              // [6]
    return;
  }

  // ---- compute waves (threads 0 .. kChainCT - 1; the mask tells the
  // compiler so, which keeps the per-thread index arithmetic branch-free).
  // Compute wave w = 2 kh + th takes k steps 2 kh, 2 kh + 1 of every slice
  // (tokens 32 kh .. 32 kh + 31) for n tiles th NT/2 .. th NT/2 + NT/2 - 1:
  // its products for different tiles are independent, and each x fragment
  // is scaled by two waves instead of four. Waves kh = 1 so hold partial
  // states over their half of the tokens; they hand them to waves kh = 0
  // (the decay scaling is linear, so it applies to the partials alike) where
  // H_c leaves, and restart from zero.
  const int ct = tid & (kChainCT - 1);
  const float Ah = A[h];
  constexpr int NT = N / 32, NH = NT / 2;
  const int th = wave & 1, kh = wave >> 1;
  // partial state, local tile u (tile t = th NH + u): n = 32 t + 8 (r / 4) + 4 g2 + r % 4, p = 32 pb + l32
  f32x16 acc[NH];
#pragma unroll
  for (int u = 0; u < NH; ++u) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n = 32 * (th * NH + u) + 8 * (r / 4) + 4 * g2 + r % 4;
      acc[u][r] = init && kh == 0 ? init[(size_t(bh) * N + n) * P + PB * pb + l32] : 0.f;
    }
  }
  // copy addresses: a uniform slice base plus this lane's 32-bit element
  // offset. Copy j of B covers rows rB0 + j (256 / RBB) of the slice (64
  // lanes x 16 bytes of RBB-chunk rows; the row swizzle is the same for
  // every j); the x copy covers rows rX.
  static_assert((256 / RBB) % 4 == 0, "copies keep the row swizzle");
  const int rB0 = (64 * wave + lane) / RBB;
  const int cB = 8 * ((lane % RBB) ^ lds_swz<RBB>(rB0));
  const int rX = (64 * wave + lane) / RBX, cX = 8 * ((64 * wave + lane) % RBX);
  const int offB = rB0 * G * N + cB, stepB = (256 / RBB) * G * N;
  const int offX = rX * H * P + cX;
  auto issue = [&](int k, int s) {
    k = min(k, nsl - 1);
    const ChunkRows cr = chunk_rows(nullptr, b, k / SPC, T, Q);
    const int s0 = (k % SPC) * kChainSK;
    const long row0 = cr.r0 + s0;
    const uint16_t* bbase = Bm + (row0 * G + g) * size_t(N);
    const uint16_t* xbase = x + (row0 * H + h) * size_t(P) + PB * pb;
    if (s0 + kChainSK <= cr.n) {                 // uniform: every row is a token of the row
#pragma unroll
      for (int j = 0; j < NCB / 4; ++j)
        copy_to_lds16(bbase + unsigned(offB + j * stepB), slotB(s) + 512 * (wave + 4 * j));
      copy_to_lds16(xbase + unsigned(offX), slotX(s) + 512 * wave);
    } else {
      // the row's last chunk: rows past its last token repeat that token.
      // rmax is negative for a slice that starts past the last token, so the
      // offsets here are signed.
      const int rmax = cr.n - 1 - s0;
#pragma unroll
      for (int j = 0; j < NCB / 4; ++j)
        copy_to_lds16(bbase + (long(min(rB0 + j * (256 / RBB), rmax)) * G * N + cB),
                      slotB(s) + 512 * (wave + 4 * j));
      copy_to_lds16(xbase + (long(min(rX, rmax)) * H * P + cX), slotX(s) + 512 * wave);
    }
  };
  // partials of waves kh = 1 handed to waves kh = 0 through a free slot,
  // fp32 in fragment order (register r of tile t of lane L at (16 t + r) 64
  // + L: lanes consecutive, no bank conflicts)
  static_assert(PB * N * 4 == kChainSK * N * 2, "an fp32 state fills one B slot");
  auto hand_over = [&](float* scr) {
#pragma unroll
    for (int u = 0; u < NH; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        scr[(16 * (th * NH + u) + r) * 64 + lane] = acc[u][r];
        acc[u][r] = 0.f;
      }
  };
  auto take_over = [&](const float* scr) {
#pragma unroll
    for (int u = 0; u < NH; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[u][r] += scr[(16 * (th * NH + u) + r) * 64 + lane];
  };
  // chunk c's start (scratch: the free slot): H_c into sH as bf16 for the
  // store waves, cumulative sums and w_s of the chunk, then the running
  // state scaled by the chunk's decay
  auto chunk_start = [&](int c, float* scr) {
    if (kh == 1) hand_over(scr);
    const float d = ct < Q ? sdtq[c & 1][ct] : 0.f;
    float v = d * Ah;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(v, off, 64);
      if (lane >= off) v += o;
    }
    if (lane == 63) sred[wave] = v;
    lds_barrier();                              // [1] partials of kh = 1 in scratch
    if (kh == 0) {
      take_over(scr);                           // acc = H_c for this wave's tiles
#pragma unroll
      for (int u = 0; u < NH; ++u) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = 32 * (th * NH + u) + 8 * j + 4 * g2;
          *reinterpret_cast<u32x2*>(&sH[l32 * kHS + n]) =
              u32x2{pack_bf16x2(acc[u][4 * j], acc[u][4 * j + 1]), pack_bf16x2(acc[u][4 * j + 2], acc[u][4 * j + 3])};
        }
      }
    }
    for (int w = 0; w < wave; ++w) v += sred[w];
    if (ct < Q) {
      sacs[ct] = v;
      sdt[ct] = d;
    }
    lds_barrier();                              // [2] sacs, sdt = chunk c; scratch read
    if (ct < Q) sw[ct] = exp_fast(sacs[Q - 1] - sacs[ct]) * sdt[ct];
    const float a = expf(sacs[Q - 1]);
#pragma unroll
    for (int u = 0; u < NH; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[u][r] *= a;
    lds_barrier();                              // [3] sH = H_c, sw = chunk c
  };
  // slice k from slot s: k steps 2 kh, 2 kh + 1, this wave's tiles
  auto compute = [&](int k, int s) {
    // padding steps past the last slice multiply by zero weights (no branch:
    // the copies and waits keep one fixed pattern)
    const float live = k < nsl ? 1.f : 0.f;
    const int s0 = (k % SPC) * kChainSK;
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      const int kb = 16 * (2 * kh + kq) + 8 * g2;
      const u32x4 xr = frag_tr<RBX>(slotX(s), kb, kb + 4, 0, lane);   // x rows kb .. kb+7 of column l32
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(&sw[s0 + kb]) * live;
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(&sw[s0 + kb + 4]) * live;
      const u32x4 a = u32x4{pack_bf16x2(bf16_lo(xr[0]) * w0[0], bf16_hi(xr[0]) * w0[1]),
                            pack_bf16x2(bf16_lo(xr[1]) * w0[2], bf16_hi(xr[1]) * w0[3]),
                            pack_bf16x2(bf16_lo(xr[2]) * w1[0], bf16_hi(xr[2]) * w1[1]),
                            pack_bf16x2(bf16_lo(xr[3]) * w1[2], bf16_hi(xr[3]) * w1[3])};
#pragma unroll
      for (int u = 0; u < NH; ++u)
        acc[u] = mfma32x32x16(frag_tr<RBB>(slotB(s), kb, kb + 4, 32 * (th * NH + u), lane), a, acc[u]);
    }
  };

  issue(0, 0);
  issue(1, 1);
  lds_barrier();                                // [0] dt of chunks 0 and 1 in sdtq
  static_assert(kChainStages == 3 && kChainSK == 64, "slot rotation and k split below");
  // whole groups of three steps (padding steps past the last slice only
  // copy), so every iteration issues the same copies in the same order
  for (int k0 = 0; k0 < nsl; k0 += 3) {
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      const int k = k0 + d;
      wait_vmcnt<OPS>();                        // this wave's copies of slice k are in
      lds_barrier();                            // [4] everyone's are; slice k - 1 is consumed
      const int sn = (d + 2) % 3;               // the slot slice k - 1 used: free
      if (k < nsl && k % SPC == 0) chunk_start(k / SPC, reinterpret_cast<float*>(slotB(sn)));
      issue(k + kChainStages - 1, sn);
      compute(k, d);
    }
  }
  wait_vmcnt<0>();                              // the last (repeated) copies
  // final = the sum of the partials
  lds_barrier();                                // [5] every slot free
  float* scr = reinterpret_cast<float*>(slotB(0));
  if (kh == 1) hand_over(scr);
  lds_barrier();                                // [6]
  if (kh == 0 && fin) {
    take_over(scr);
#pragma unroll
    for (int u = 0; u < NH; ++u) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = 32 * (th * NH + u) + 8 * (r / 4) + 4 * g2 + r % 4;
        fin[(size_t(bh) * N + n) * P + PB * pb + l32] = acc[u][r];
      }
    }
  }
}

template <int N, int P, int SPC>
hipError_t launch_chain_np(const FwdShape& s, const void* x, const void* B, const void* C, const void* dt,
                           const float* A, float* Acs, float* dtq, uint16_t* Hb, const float* init, float* fin,
                           uint16_t* CB, hipStream_t st, const StageEv& ev) {
  const int lpc = s.Q / 32;
  const long ntiles = long(s.b) * s.nc * s.G * (lpc * (lpc + 1) / 2);
  const long nchain = long(s.b) * s.H * (P / 32);
  const long blocks = nchain + (ntiles + kChainWaves - 1) / kChainWaves;
  hipExtLaunchKernelGGL((chunk_state_chain_kernel<N, P, SPC>), dim3(unsigned(blocks)), dim3(kChainThreads), 0, st,
                        ev.start, ev.stop, 0, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(B),
                        static_cast<const uint16_t*>(dt), A, Acs, dtq, Hb, init, fin,
                        static_cast<const uint16_t*>(C), CB, s.T, s.H, s.G, s.Q, s.nc, int(nchain), ntiles);
  return hipGetLastError();
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

template <int N_, int P_>
struct ChainNP {
  static constexpr int n = N_, p = P_;
};

// The fused launch pays off when its chains fill the chip in one round: each
// chain is a serial walk over its row's slices, so fewer chains than
// compute units leave units idle and more than fit at once (two work-groups
// per unit at dstate 128, one at 256 for their local memory) run in two
// rounds of the whole walk; such shapes take the two-kernel path.
bool chunk_state_chain_ok(const FwdShape& s) {
  if (!((s.N == 128 || s.N == 256) && (s.P == 32 || s.P == 64 || s.P == 128) && s.Q % kChainSK == 0)) return false;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return false;
  const long chains = long(s.b) * s.H * (s.P / 32);
  const long per_cu = s.N == 128 ? 2 : 1;
  return chains >= cus && chains <= per_cu * cus;
}

hipError_t launch_chunk_state_chain(const FwdShape& s, const void* x, const void* B, const void* C,
                                    const void* dt, const float* A, float* Acs, float* dtq, uint16_t* Hb,
                                    const float* init, float* fin, uint16_t* CB, hipStream_t st,
                                    const StageEv& ev) {
  if (!chunk_state_chain_ok(s)) return hipErrorInvalidValue;
  auto by_q = [&](auto np) -> hipError_t {
    using NP = decltype(np);
    switch (s.Q / kChainSK) {
      case 1: return launch_chain_np<NP::n, NP::p, 1>(s, x, B, C, dt, A, Acs, dtq, Hb, init, fin, CB, st, ev);
      case 2: return launch_chain_np<NP::n, NP::p, 2>(s, x, B, C, dt, A, Acs, dtq, Hb, init, fin, CB, st, ev);
      case 4: return launch_chain_np<NP::n, NP::p, 4>(s, x, B, C, dt, A, Acs, dtq, Hb, init, fin, CB, st, ev);
    }
    return hipErrorInvalidValue;
  };
  if (s.N == 128) {
    if (s.P == 32) return by_q(ChainNP<128, 32>{});
    if (s.P == 64) return by_q(ChainNP<128, 64>{});
    return by_q(ChainNP<128, 128>{});
  }
  if (s.P == 32) return by_q(ChainNP<256, 32>{});
  if (s.P == 64) return by_q(ChainNP<256, 64>{});
  return by_q(ChainNP<256, 128>{});
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
