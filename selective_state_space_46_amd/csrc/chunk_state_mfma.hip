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
#include <algorithm>
#include <atomic>

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
// BOTH (the backward's recomputation): the tiles stay fp32 (4 KB per tile at
// the same index, as four 1 KB rows of 64 float4: quad m of lane L at float4
// 64 m + L, so that a 16-byte load per lane reads one whole row), and the
// same products with the roles of the two operands swapped go to CBt, where
// lane L holds column s = L%32 and the registers run over rows l. The
// backward takes sums of these products that largely cancel, so they are not
// rounded to bf16.
// The C rows of 32-row block i of chunk (b, c), group g, as this lane holds
// them for the matrix cores (cf[ks]: row 32 i + L % 32, dstate 16 ks + 8 (L /
// 32) .. + 7; zeros past the chunk's tokens), stored in that order:
// CF [b, nc, G, Q / 32, N / 16, 64 lanes, 8] bf16, so that chunk_scan reads
// each operand as one contiguous 1 KB per wave (from C itself each of its
// loads reads 32 bytes in each of 32 rows).
template <int N>
__device__ __forceinline__ void store_c_frags(uint16_t* __restrict__ CF, const u32x4 (&cf)[N / 16], int b, int c,
                                              int g, int i, int G, int Q, int nc, int lane) {
  u32x4* dst = reinterpret_cast<u32x4*>(CF) + (((size_t(b) * nc + c) * G + g) * (Q / 32) + i) * (N / 16) * 64 + lane;
#pragma unroll
  for (int ks = 0; ks < N / 16; ++ks) dst[64 * ks] = cf[ks];
}

template <int N, bool BOTH = false>
__device__ __forceinline__ void chunk_scores_tile(const uint16_t* __restrict__ Bm,
                                                  const uint16_t* __restrict__ Cm,
                                                  uint16_t* __restrict__ CB, uint16_t* __restrict__ CBt,
                                                  const int4* __restrict__ tab, int T, int G, int Q, int nc,
                                                  long wid, int lane, uint16_t* __restrict__ CF = nullptr) {
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
  const size_t tile_at = (((size_t(b) * nc + c) * G + g) * ntile + ti) * 1024;
  const size_t at = tile_at + size_t(lane) * 16;
  if (CF && j == 0) store_c_frags<N>(CF, cf, b, c, g, i, G, Q, nc, lane);
  auto store32 = [&](uint16_t* dstbase, const f32x16& acc) {
    f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(dstbase) + tile_at) + lane;
#pragma unroll
    for (int m = 0; m < 4; ++m) dst[64 * m] = f32x4{acc[4 * m], acc[4 * m + 1], acc[4 * m + 2], acc[4 * m + 3]};
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
    const int4* __restrict__ tab, int T, int H, int G, int Q, int nc, int nscore_wg, long ntiles,
    uint16_t* __restrict__ CF) {
  // the first nscore_wg work-groups compute C B^T tiles, one per wave (and
  // with CF, C in chunk_scan's operand order)
  if (int(blockIdx.x) < nscore_wg) {
    const long wid = long(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (wid < ntiles)
      chunk_scores_tile<N, MODE == 1>(Bm, Cm, CB, CBt, tab, T, G, Q, nc, wid, threadIdx.x & 63, CF);
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
// steps 2 and 3). A work-group owns one batch row and CW (64 or 128, see
// chain_cols) consecutive columns of the flattened (head, p) axis -- 32-column
// blocks of one head, or of two heads in one B/C group -- and walks that
// row's chunks in
// order, its running states held in the fp32 accumulators of the matrix
// cores: at a chunk's start the accumulators (= H_c) go out as bf16 for
// chunk_scan, are scaled by the chunk's decay, and the chunk's products then
// accumulate on top, leaving H_{c+1}. The fp32 chunk states S_c never reach
// HBM (the two-kernel form writes and re-reads them).
//
// Segments (forward only). Where one walk per (batch row, CW columns) leaves
// most compute units idle (a few long rows), each row is cut into nseg
// segments of seglen consecutive chunks (the last may be shorter) and every
// (row, CW columns, segment) walks its own segment: segment 0 from the
// initial state, the others from zero. The state handed from chunk to chunk
// is linear in the state a segment starts from, and the summaries compose
// associatively ((decay_1, S_1) then (decay_2, S_2) gives (decay_1 decay_2,
// decay_2 S_1 + S_2); youngju.dev "Mamba / selective SSM",
// "SSDアルゴリズムとチャンク分割": the state passed between chunks by the
// recurrence), so the true state entering chunk c of segment k is
//   H_c = H_c^local + exp(cdec_c) Hin_k,
// with cdec_c the summed chunk decay exponents from the segment's start to c
// and Hin_k the state entering segment k. A segmented walk writes H_c^local
// (bf16), cdec (fp32 [b, H, nc]), its segment's total decay exponent (segdec,
// fp32 [b, H, nseg]) and its last local state (fp32 [b, nseg, H, P * N] in
// fragment order, as the bf16 states) in place of the final state;
// state_passing then runs the recurrence over the segments, and chunk_scan
// adds exp(cdec_c) Hin_k where it stages H_c.
//
// Packed sequences (vw.tab not null): one row of chunk slots (the chunk table
// gives each slot's rows, sequence and whether it begins or ends its
// sequence) cut into equal segments like a batch row. A walk starts from
// zero and, at each chunk that begins a sequence, restarts from that
// sequence's initial state; the state handed from chunk to chunk is reset
// there (youngju.dev page, "状態初期化とシーケンス境界": no state crosses from
// one sequence into the next). From the first restart on, cdec is -inf (no
// chunk after it takes the state entering the segment) and so is segdec (no
// state passes through the segment). At the end of a sequence's last chunk
// the running state is its final state if the sequence began inside this
// walk; if it is the segment's first sequence, continued from before, it is
// its local end state, left in F with its decay exponent (fdec) and the
// sequence (fseq) for the recurrence over segments. Unused slots (between
// sequences) have no rows: zero weights and decay 1 leave the state as it is.
//
// Tokens stream through 64-row slices of B (all of dstate, shared by the
// column blocks) and x (the CW columns), copied straight from global memory
// into LDS (global_load_lds, 16 bytes per lane) in a swizzled row-major
// layout, STAGES slices resident: one read while the others load. The copies
// use no registers. The MFMA operands are read transposed
// (ds_read_b64_tr_b16); the x fragment is scaled by
// w_s = exp(Acs_{Q-1} - Acs_s) dt_s there and rounded to bf16 once (the same
// W = w x as chunk_state_mfma_kernel). The product is taken as S[n][p] (rows
// n, lanes p), so a lane holds four consecutive n of one p: H_c leaves as
// runs of its [p][n] rows, init and final ([n][p]) as whole rows of p.
//
// Waves: two compute waves per 32-column block (CW / 16 in all; wave w:
// column block w % (CW / 32), n tiles w / (CW / 32), that + 2, ...), one
// table wave and three copy waves. The table wave
// builds each chunk's weights and decay one chunk ahead from dt loaded one
// chunk before that, and writes the Acs / dt rows; the copy waves issue the
// slice copies and wait for them by count. The vector memory counter counts
// loads and stores together, and a wait the compiler places for a register
// load covers everything issued after it, so each kind of memory work sits
// in a wave of its own: the copy waves hold nothing but copies, the table
// wave's dt loads are a chunk old when used, and the compute waves only
// store. All waves pass the same barriers, one per slice.
// ---------------------------------------------------------------------------
constexpr int kChainWaves = 8;      // waves of a C B^T tile work-group (one tile per wave)
constexpr int kChainThreads = 64 * kChainWaves;
constexpr int kChainSK = 64;        // tokens per slice
constexpr int kVarWalkSlots = 128;  // chunk slots per walk over packed rows (at most)

// Columns per work-group. The forward at dstate 256, headdim 64 and
// chunk_len 256 (spc = 4 slices per chunk) takes 128: each 32 KB slice of B
// then serves twice the columns (B moves from L2 into LDS once per 128
// columns instead of per 64), with eight compute waves (4 column blocks x 2
// n-tile groups), 12 waves in all and 150 KB of LDS. Elsewhere 64 (the
// backward's walks; dstate 128, whose slices are half the size; other
// headdims and shorter chunks, whose per-head and chunk-start work does not
// fit the 168 registers a wave of 12 has).
constexpr int chain_cols(int N, int P, int spc, bool bwd) {
  return N == 256 && P == 64 && spc == 4 && !bwd ? 128 : 64;
}
// waves of a work-group: 2 per 32-column block (compute), 1 table, 3 copy
constexpr int chain_waves(int cols) { return cols / 16 + 4; }

template <int V>
struct IntC {
  static constexpr int value = V;
};

// ST slices resident: 5 at dstate 128 (120 KB: one work-group per compute
// unit), 3 there when two work-groups share a unit (72 KB each), 3 at
// dstate 256 (120 KB)
template <int N, int ST, int CW>
struct ChainCfg {
  static constexpr int STAGES = ST;
  static constexpr int RBB = N / 8, RBX = CW / 8;                // 16-byte chunks per B / x row
  static constexpr int NCB = kChainSK * RBB / 64, NCX = kChainSK * RBX / 64;   // wave copies per slice
  static constexpr int OPS = (NCB + NCX + 2) / 3;                // copies per copy wave and slice
  static constexpr int TPW = N / 64;                             // n tiles per compute wave
  static_assert((STAGES - 2) * OPS < 64, "copies in flight fit the counter");
};

// F32S (the backward's recomputation): the states entering each chunk go
// out as fp32 ([b, c, h, p, n], as state_passing leaves them over the chunk
// states) and the C B^T tiles as fp32 in both orientations (CB and CBt, as
// chunk_state_mfma_kernel's MODE 1); else bf16 states and bf16 tiles.
//
// REV (the backward's reverse pass): the same walk over the chunks in
// reverse order with x -> dy, B -> C and the token weights exp(Acs_l) (the
// chunk's inclusive cumulative decay), which carries the gradient G_c of the
// state leaving chunk c backwards: G_{nc-1} = dfinal (init),
// G_{c-1} = exp(Acs_c[Q-1]) G_c + sum_l exp(Acs_l) C_l dy_l^T, d init = G_{-1}
// (fin). Each G_c goes out as bf16 in Hs ([b, c, h, p, n]) with its dot
// products with H_c (fp32 states entering each chunk, Hst) in per-wave
// partials: ghp[((b H + h) nc + c) P / 16 + part]. No tiles, Acs or dt rows.
template <int N, int P, int SPC, int ST, bool F32S, bool REV, bool VAR>
__global__ __launch_bounds__(64 * chain_waves(chain_cols(N, P, SPC, F32S || REV)))
__attribute__((amdgpu_waves_per_eu(N == 128 && ST <= 3 ? 4 : 1)))
void chunk_state_chain_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ dt,
    const float* __restrict__ A, float* __restrict__ Acs, float* __restrict__ dtq, void* __restrict__ Hs,
    const float* __restrict__ init, float* __restrict__ fin, const uint16_t* __restrict__ Cm,
    uint16_t* __restrict__ CB, uint16_t* __restrict__ CBt, const float* __restrict__ Hst, float* __restrict__ ghp,
    float* __restrict__ cdec, float* __restrict__ segdec, int T, int H, int G, int Q, int nc, int nb, int nseg,
    int seglen, int nchain, long ntiles, VarWalk vw, uint16_t* __restrict__ CF) {
  constexpr int CW = chain_cols(N, P, SPC, F32S || REV);   // columns per work-group
  constexpr int NCOLB = CW / 32;                // 32-column blocks
  constexpr int NCWV = 2 * NCOLB;               // compute waves; the table wave is wave NCWV
  constexpr int NW = chain_waves(CW), NTHR = 64 * NW;
  using Cfg = ChainCfg<N, ST, CW>;
  constexpr int S = Cfg::STAGES, RBB = Cfg::RBB, RBX = Cfg::RBX, NCB = Cfg::NCB, NCX = Cfg::NCX;
  constexpr int OPS = Cfg::OPS, TPW = Cfg::TPW;
  constexpr int NHW = P < CW ? CW / P : 1;      // heads per work-group
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = wave_id();  // wave-uniform (scalar register)
  // work-groups past the chains compute C B^T tiles, one per wave
  if (int(blockIdx.x) >= nchain) {
    const long wid = long(int(blockIdx.x) - nchain) * NW + wave;
    if (wid < ntiles) chunk_scores_tile<N, F32S>(Bm, Cm, CB, CBt, nullptr, T, G, Q, nc, wid, lane, CF);
    return;                                     // no barrier on this path
  }
  __shared__ __attribute__((aligned(16))) uint16_t sB[S][kChainSK * N];
  __shared__ __attribute__((aligned(16))) uint16_t sX[S][kChainSK * CW];
  // chunk c's token weights w_s = exp(Acs_{Q-1} - Acs_s) dt_s and decay
  // exp(Acs_{Q-1}) of head h0 + q in [q][c & 1]
  __shared__ __attribute__((aligned(16))) float sw[NHW][2][kMaxQ];
  __shared__ float sdecay[NHW][2];
  // packed rows: the walk's chunk table entries {first row, valid tokens,
  // sequence, flags}, clamped (first row in [0, T), sequence in [0, nseq)),
  // read once from global memory: the waves then take rows, flags and
  // sequences from LDS, so no global load joins the copy waves' counted
  // copies
  __shared__ int4 sslot[kVarWalkSlots];

  // walk id = ((b nseg + seg) cpr + column block): the walks of one (row,
  // segment) share every B slice and sit next to each other (one XCD's L2)
  const int id = xcd_swizzle(int(blockIdx.x), nchain);
  const int cpr = H * P / CW;                   // work-groups per batch row and segment
  const int c0 = (id % cpr) * CW;               // first flattened column
  const int seg = (id / cpr) % nseg, b = id / cpr / nseg;
  const int h0 = c0 / P;                        // first head
  const int g = h0 / (H / G);                   // the B group (both heads share it)
  const int l32 = lane & 31, g2 = lane >> 5;
  const int cbeg = seg * seglen;                // first chunk of the walk
  const int ncw = min(nc, cbeg + seglen) - cbeg;   // chunks of the walk
  const int nsl = ncw * SPC;                    // slices of the walk
  constexpr bool var = VAR;                     // packed rows (vw.tab not null)
  if (var) {
    // ncw <= seglen <= kVarWalkSlots (the launcher checks)
    for (int t = tid; t < ncw; t += NTHR) {
      const int4 e = vw.tab[cbeg + t];
      const int r0 = clamp_int(e.x, 0, T - 1);
      sslot[t] = int4{r0, clamp_int(min(e.y, T - r0), 0, Q), clamp_int(e.z, 0, vw.nseq - 1), e.w};
    }
    __syncthreads();                            // uniform: var is
  }
  // token rows of chunk c: equal-length rows, or the chunk table's slot (an
  // unused slot has none: its loads read one clamped row, its weights are 0)
  auto rows = [&](int c) {
    if (var) {
      const int4 e = sslot[c - cbeg];
      return ChunkRows{long(e.x), e.y};
    }
    return chunk_rows(nullptr, b, c, T, Q);
  };
  // the walk's step k visits slice ks(k) of the row and its chunk wc = k / SPC
  // is chunk rc(wc) of the row (reversed in the reverse pass)
  auto ks = [&](int k) { return REV ? (cbeg + ncw) * SPC - 1 - k : cbeg * SPC + k; };
  auto rc = [&](int wc) { return REV ? cbeg + ncw - 1 - wc : cbeg + wc; };
  const size_t hstate = size_t(P) * N;          // elements of one (b, h) state
  // whether this work-group holds the first columns of each of its heads
  // (they write the per-head rows: Acs, dt, cdec, segdec); a head wider
  // than the work-group is split over several
  const bool hfirst = P < CW || c0 % P == 0;

  if (wave == NCWV) {
    // ---- table wave: each chunk's tables one chunk ahead, from dt loaded one
    // chunk before that. It issues no copies, so its loads (dt) and stores
    // (the Acs / dt rows) are all its memory counter holds: the wait for a
    // chunk's dt finds only operations a chunk old.
    float Ah[NHW];
#pragma unroll
    for (int q = 0; q < NHW; ++q) Ah[q] = A[h0 + q];
    // dt of tokens 4 lane .. 4 lane + 3 of chunk c, head h0 + q (rows clamped
    // into the row; the tables zero those past its end), each as the aligned
    // 32-bit word of the tensor that holds it (dt is 16-byte aligned, so the
    // word of element e starts at e & ~1) and, in bit i of hi, whether it is
    // that word's upper half. 32-bit loads need no widening, which would wait
    // for them at once. The one exception is the tensor's last element when
    // its index is even: its word would end past the tensor, so it is read
    // alone (16 bits, in the low half). Only the chunk that holds the
    // tensor's last token row, in the work-group that holds its last head,
    // can meet it; that case is a separate, uniform branch, so every other
    // chunk's loads are whole aligned words.
    const long last_e = long(nb) * T * H - 1;   // the tensor's last element
    auto dt_load = [&](int wc, uint32_t (&v)[NHW][4], uint32_t (&hi)[NHW]) {
      const ChunkRows cr0 = rows(rc(wc));
      // rows read: r0 .. r0 + nr - 1 (r0 < T and at least one row, also for
      // an unused slot of a packed row)
      const ChunkRows cr = ChunkRows{min(cr0.r0, long(nb) * T - 1), max(cr0.n, 1)};
      const bool tail = (last_e & 1) == 0 && cr.r0 + cr.n == long(nb) * T && h0 + NHW == H;
      if (tail) {
#pragma unroll
        for (int q = 0; q < NHW; ++q) {
          hi[q] = 0u;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const long e = (cr.r0 + min(4 * lane + i, cr.n - 1)) * H + h0 + q;
            const uint32_t up = uint32_t(e & 1);
            v[q][i] = e == last_e ? uint32_t(dt[e]) : *reinterpret_cast<const uint32_t*>(dt + (e - up));
            hi[q] |= up << i;
          }
        }
        return;
      }
#pragma unroll
      for (int q = 0; q < NHW; ++q) {
        hi[q] = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const long e = (cr.r0 + min(4 * lane + i, cr.n - 1)) * H + h0 + q;
          const uint32_t up = uint32_t(e & 1);
          v[q][i] = *reinterpret_cast<const uint32_t*>(dt + (e - up));
          hi[q] |= up << i;
        }
      }
    };
    // chunk c's tables for head h0 + q (four tokens per lane: a serial sum per
    // lane and one wave scan of the lane totals) into slot c & 1; Acs and dt
    // of this lane's tokens into acs / v for the rows written after the next
    // dt loads
    auto tables = [&](int wc, int q, const uint32_t (&raw)[4], uint32_t hi, float (&acs)[4], float (&v)[4]) -> float {
      const ChunkRows cr = rows(rc(wc));
      float tot = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t bits = (hi >> i) & 1 ? raw[i] & 0xffff0000u : raw[i] << 16;
        v[i] = 4 * lane + i < cr.n ? __uint_as_float(bits) : 0.f;
        tot += v[i] * Ah[q];
      }
      float run = wave_incl_scan(tot) - tot;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        run += v[i] * Ah[q];
        acs[i] = run;
      }
      // Acs_{Q-1}: element (Q - 1) % 4 of lane (Q - 1) / 4 (Q is a multiple of 64)
      const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acs[3]), (Q - 1) / 4));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * lane + i < Q)
          sw[q][wc & 1][4 * lane + i] =
              REV ? (4 * lane + i < cr.n ? exp_fast(acs[i]) : 0.f) : exp_fast(last - acs[i]) * v[i];
      if (lane == 0) sdecay[q][wc & 1] = expf(last);
      return last;
    };
    // the Acs / dt rows of chunk c, head h0 + q (by the work-group holding
    // the head's first columns)
    auto rows_out = [&](int c, int q, const float (&acs)[4], const float (&v)[4]) {
      if (!hfirst) return;
      const size_t arow = ((size_t(b) * H + h0 + q) * nc + c) * Q;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * lane + i;
        if (t < Q) {
          Acs[arow + t] = acs[i];
          dtq[arow + t] = v[i];
        }
      }
    };
    uint32_t dnext[NHW][4], dhi[NHW];
#pragma unroll
    for (int q = 0; q < NHW; ++q) {
      dhi[q] = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) dnext[q][i] = 0u;
    }
    float tacs[NHW][4], tdt[NHW][4];
    // segmented walks: the summed decay exponents of the segment's chunks
    // before chunk c (cdec), and of all its chunks (segdec), per head, by the
    // work-group that holds the head's first columns
    float run[NHW];
#pragma unroll
    for (int q = 0; q < NHW; ++q) run[q] = 0.f;
    // packed rows: a sequence has begun inside this walk (from then on no
    // chunk takes the state entering the segment: cdec, segdec -inf); the
    // segment's first sequence is none until its end is seen
    bool dead = false;
    const bool lead = var && c0 == 0 && lane == 0;   // writes fseq[seg]
    if (lead && vw.fseq) vw.fseq[seg] = -1;
    // chunk c's tables, then chunk c + 1's dt, then chunk c's rows (stores
    // after the loads)
    auto chunk = [&](int wc) {
      float lastq[NHW];
#pragma unroll
      for (int q = 0; q < NHW; ++q) lastq[q] = tables(wc, q, dnext[q], dhi[q], tacs[q], tdt[q]);
      if (wc + 1 < ncw) dt_load(wc + 1, dnext, dhi);
      if constexpr (!REV) {
        int flags = 0, sqc = 0;
        if (var) {
          const int4 e = sslot[wc];
          flags = e.w;
          sqc = e.z;
          if (flags & 1) dead = true;           // a sequence begins at this chunk
        }
#pragma unroll
        for (int q = 0; q < NHW; ++q) {
          rows_out(rc(wc), q, tacs[q], tdt[q]);
          if (cdec && hfirst && lane == 0)
            cdec[(size_t(b) * H + h0 + q) * nc + rc(wc)] = dead ? -INFINITY : run[q];
          run[q] += lastq[q];
          // the segment's first sequence, continued from before, ends here:
          // its decay exponent from the segment's start through this chunk
          if (var && (flags & 2) && !dead && hfirst && lane == 0 && vw.fdec)
            vw.fdec[size_t(h0 + q) * nseg + seg] = run[q];
        }
        if (var && (flags & 2) && !dead && lead && vw.fseq) vw.fseq[seg] = sqc;
      }
    };
    dt_load(0, dnext, dhi);
    chunk(0);
    for (int k0 = 0; k0 < nsl; k0 += S) {
#pragma unroll
      for (int d = 0; d < S; ++d) {
        const int k = k0 + d;
        lds_barrier();                          // [4]
        // at chunk c's start, chunk c + 1's tables (slot (c + 1) & 1 last
        // served chunk c - 1, whose slices are consumed by now; the compute
        // waves read it one barrier later at the earliest)
        if (k < nsl && k % SPC == 0 && k / SPC + 1 < ncw) chunk(k / SPC + 1);
      }
    }
    if (segdec) {
#pragma unroll
      for (int q = 0; q < NHW; ++q)
        if (hfirst && lane == 0) segdec[(size_t(b) * H + h0 + q) * nseg + seg] = dead ? -INFINITY : run[q];
    }
    return;
  }

  if (wave > NCWV) {
    // ---- copy waves: the slice copies into LDS. Copy q of a slice (q < NCB:
    // B, else x) covers 1 KB of its slot; copy wave v takes q = v, v + 3, ...,
    // the last index repeated where the count falls short (the repeat writes
    // the same bytes again). Each copy wave's loop is compiled for its own
    // copies, so a copy is a uniform slice base plus a per-lane offset
    // computed once.
    auto copy_loop = [&](auto svc) {
      constexpr int SV = decltype(svc)::value;
      // lane offsets (elements) of this wave's copies inside a whole slice:
      // B rows q (512 / N) + lane / RBB, x rows qx (512 / 64) + lane / RBX,
      // each lane fetching the 16-byte chunk the swizzle places at its LDS
      // position; and the rows, for the clamped copies of a partial slice
      unsigned off[OPS];
      int row[OPS], cc[OPS];
#pragma unroll
      for (int i = 0; i < OPS; ++i) {
        const int q = min(SV + 3 * i, NCB + NCX - 1);
        if (q < NCB) {
          row[i] = q * (512 / N) + lane / RBB;
          cc[i] = 8 * ((lane % RBB) ^ lds_swz<RBB>(row[i]));
          off[i] = unsigned(row[i] * G * N + cc[i]);
        } else {
          row[i] = (q - NCB) * (512 / CW) + lane / RBX;
          cc[i] = 8 * ((lane % RBX) ^ lds_swz<RBX>(row[i]));
          off[i] = unsigned(row[i] * H * P + cc[i]);
        }
      }
      // slice k (clamped into the row: copies past its end repeat the last
      // slice into a free slot) into slot s
      auto issue = [&](int k, int s) {
        k = ks(min(k, nsl - 1));
        const ChunkRows cr0 = rows(k / SPC);
        // at least one row read, inside the tensor (an unused slot of a packed
        // row reads one clamped row; its weights are zero)
        const ChunkRows cr = ChunkRows{min(cr0.r0, long(nb) * T - 1), max(cr0.n, 1)};
        const int s0 = (k % SPC) * kChainSK;
        const long row0 = cr.r0 + s0;
        const uint16_t* bbase = Bm + (row0 * G + g) * size_t(N);
        const uint16_t* xbase = x + row0 * size_t(H) * P + c0;
        if (s0 + kChainSK <= cr.n) {            // uniform: every row is a token of the row
#pragma unroll
          for (int i = 0; i < OPS; ++i) {
            const int q = min(SV + 3 * i, NCB + NCX - 1);
            if (q < NCB) copy_to_lds16(bbase + off[i], &sB[s][512 * q]);
            else copy_to_lds16(xbase + off[i], &sX[s][512 * (q - NCB)]);
          }
        } else {
          // rows past the row's last token repeat that token (rmax is
          // negative for a slice that starts past it: signed offsets)
          const int rmax = cr.n - 1 - s0;
#pragma unroll
          for (int i = 0; i < OPS; ++i) {
            const int q = min(SV + 3 * i, NCB + NCX - 1);
            if (q < NCB)
              copy_to_lds16(bbase + (long(min(row[i], rmax)) * G * N + cc[i]), &sB[s][512 * q]);
            else
              copy_to_lds16(xbase + (long(min(row[i], rmax)) * H * P + cc[i]), &sX[s][512 * (q - NCB)]);
          }
        }
      };
#pragma unroll
      for (int k = 0; k < S - 1; ++k) issue(k, k);
      // Slice k's copies were issued S - 1 steps earlier; this wave's copies
      // complete in order, so waiting until at most the S - 2 slices issued
      // after it (OPS copies each) are outstanding leaves slice k in LDS.
      for (int k0 = 0; k0 < nsl; k0 += S) {
#pragma unroll
        for (int d = 0; d < S; ++d) {
          const int k = k0 + d;
          wait_vmcnt<(S - 2) * OPS>();
          lds_barrier();                        // [4] slice k in LDS; slice k - 1 consumed
          issue(k + S - 1, (d + S - 1) % S);    // into the slot slice k - 1 used
        }
      }
      wait_vmcnt<0>();                          // the last (repeated) copies
    };
    if (wave == NCWV + 1) copy_loop(IntC<0>{});
    else if (wave == NCWV + 2) copy_loop(IntC<1>{});
    else copy_loop(IntC<2>{});
    return;
  }

  // ---- compute waves (waves 0 .. NCWV - 1): 32-column block j = wave %
  // NCOLB (of head hj), n tiles wave / NCOLB + 2 u. Each owns its
  // tiles over every token, so the running states need no exchange between
  // waves; they issue no loads inside the walk, so their stores (H_c, the
  // final state) cost no waits.
  const int j = wave % NCOLB;                   // 32-column block
  const int hj = (c0 + 32 * j) / P, hq = hj - h0;   // its head
  const int pj = (c0 + 32 * j) % P;             // its first column of that head
  const size_t bhj = size_t(b) * H + hj;
  auto ntile = [&](int u) { return wave / NCOLB + 2 * u; };
  // running state, tile u: n = 32 ntile(u) + 8 (r / 4) + 4 g2 + r % 4, p = pj + l32 of head hj
  f32x16 acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n = 32 * ntile(u) + 8 * (r / 4) + 4 * g2 + r % 4;
      acc[u][r] = init && seg == 0 && !var ? init[(bhj * N + n) * P + pj + l32] : 0.f;
    }
  }
  // chunk c's start: H_c out as bf16 ([p][n] rows, four consecutive n of
  // p = pj + l32 per register run), then the running state scaled by the
  // chunk's decay
  // REV: this lane's part of H_c (fp32, the runs of the accumulator layout),
  // loaded one chunk ahead of its dot product with G_c
  f32x4 hnext[REV ? TPW * 4 : 1];
  auto h_load = [&](int c) {
    if constexpr (REV) {
      const float* hrow = Hst + ((size_t(b) * nc + c) * H + hj) * hstate + size_t(pj + l32) * N;
#pragma unroll
      for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          hnext[4 * u + jj] = *reinterpret_cast<const f32x4*>(hrow + 32 * ntile(u) + 8 * jj + 4 * g2);
    }
  };
  if constexpr (REV) h_load(rc(0));
  // packed rows: the running state is a sequence's; at its last chunk's end
  // it is that sequence's final state (restarted inside this walk: cdead) or
  // the local end state of the segment's first sequence, continued from
  // before (F, completed by the recurrence over segments)
  bool cdead = false;
  int pflag = 0, pseq = 0;                      // the previous chunk's flags and sequence
  // lane-dependent addresses recomputed at each use (see opaque): a lane's
  // elements of an [n][p] state are one lane base plus constant offsets, and
  // of a fragment-order one too (hb_off: lane part 4 (l32 + 32 g2))
  auto np_base = [&](size_t row0) {            // row0: (sequence H + head) of an [.., N, P] tensor
    const int ln = opaque(lane);
    return row0 * N * P + size_t(4 * (ln >> 5)) * P + pj + (ln & 31);
  };
  auto np_off = [&](int u, int r) { return (32 * ntile(u) + 8 * (r / 4) + r % 4) * P; };
  auto finish = [&](int sqn) {
    if (cdead) {
      if (vw.fin) {
        float* dst = vw.fin + np_base(size_t(sqn) * H + hj);
#pragma unroll
        for (int u = 0; u < TPW; ++u)
#pragma unroll
          for (int r = 0; r < 16; ++r) dst[np_off(u, r)] = acc[u][r];
      }
    } else if (vw.F) {
      const int ln = opaque(lane);
      float* dst = vw.F + (size_t(seg) * H + hj) * hstate + hb_off(pj, 0, N) + 4 * ln;
#pragma unroll
      for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *reinterpret_cast<f32x4*>(dst + hb_off(0, 32 * ntile(u) + 8 * jj, N)) =
              f32x4{acc[u][4 * jj], acc[u][4 * jj + 1], acc[u][4 * jj + 2], acc[u][4 * jj + 3]};
    }
  };
  auto chunk_start = [&](int wc) {
    const int c = rc(wc);
    if (var) {
      const int4 e = sslot[wc];
      const int f = e.w, sqc = e.z;
      if (pflag & 2) finish(pseq);              // the previous chunk ended a sequence
      if (f & 1) {
        // a sequence begins: its initial state (or zero)
        cdead = true;
        if (init) {
          const float* src = init + np_base(size_t(sqc) * H + hj);
#pragma unroll
          for (int u = 0; u < TPW; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[u][r] = src[np_off(u, r)];
        } else {
#pragma unroll
          for (int u = 0; u < TPW; ++u) acc[u] = zero16();
        }
      }
      pflag = f;
      pseq = sqc;
    }
    if constexpr (REV) {
      // <G_c, H_c>: this wave's part, one partial per wave
      float dot = 0.f;
#pragma unroll
      for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int e = 0; e < 4; ++e) dot += acc[u][4 * jj + e] * hnext[4 * u + jj][e];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
      if (lane == 0) ghp[((size_t(b) * H + hj) * nc + c) * (P / 16) + 2 * (pj / 32) + wave / NCOLB] = dot;
    }
    // fp32 (F32S) and the reverse walk's gradients: [p][n] rows; the forward's
    // bf16 states: fragment order (hb_off), the accumulators as they are
    const size_t sbase = ((size_t(b) * nc + c) * H + hj) * hstate;
    const size_t hoff = sbase + size_t(pj + l32) * N;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int n = 32 * ntile(u) + 8 * jj + 4 * g2;
        const u32x2 v2 = u32x2{pack_bf16x2(acc[u][4 * jj], acc[u][4 * jj + 1]),
                               pack_bf16x2(acc[u][4 * jj + 2], acc[u][4 * jj + 3])};
        if constexpr (F32S) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(Hs) + hoff + n) =
              f32x4{acc[u][4 * jj], acc[u][4 * jj + 1], acc[u][4 * jj + 2], acc[u][4 * jj + 3]};
        } else if constexpr (REV) {
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(Hs) + hoff + n) = v2;
        } else {
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(Hs) + sbase + hb_off(pj + l32, n, N)) = v2;
        }
      }
    }
    const float decay = sdecay[hq][wc & 1];
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[u][r] *= decay;
    // the next chunk's H (after this chunk's stores: a later wait for the
    // loads then finds only older stores)
    if (REV && wc + 1 < ncw) h_load(rc(wc + 1));
  };
  // slice k from slot s, all four k steps
  auto compute = [&](int k, int s) {
    // padding steps past the last slice (they keep the barrier pattern
    // fixed) compute nothing
    if (k >= nsl) return;
    const int s0 = (ks(k) % SPC) * kChainSK;
    const float* swc = sw[hq][(k / SPC) & 1];
    constexpr int KS = kChainSK / 16;
    // the LDS reads of KG k steps first, so that one wait covers them all:
    // the whole slice at 64 columns; two k steps at a time at 128 (12 waves
    // leave 168 registers a wave)
    constexpr int KG = CW == 128 ? 2 : KS;
#pragma unroll
    for (int kq = 0; kq < KS; kq += KG) {
      u32x4 xr[KG], bf[KG][TPW];
      f32x4 w0[KG], w1[KG];
#pragma unroll
      for (int kk = 0; kk < KG; ++kk) {
        const int kb = 16 * (kq + kk) + 8 * g2;
        xr[kk] = frag_tr<RBX>(sX[s], kb, kb + 4, 32 * j, lane);   // x rows kb .. kb+7 of column 32 j + l32
        w0[kk] = *reinterpret_cast<const f32x4*>(&swc[s0 + kb]);
        w1[kk] = *reinterpret_cast<const f32x4*>(&swc[s0 + kb + 4]);
#pragma unroll
        for (int u = 0; u < TPW; ++u) bf[kk][u] = frag_tr<RBB>(sB[s], kb, kb + 4, 32 * ntile(u), lane);
      }
#pragma unroll
      for (int kk = 0; kk < KG; ++kk) {
        const f32x4 v0 = w0[kk], v1 = w1[kk];
        const u32x4 a = u32x4{pack_bf16x2(bf16_lo(xr[kk][0]) * v0[0], bf16_hi(xr[kk][0]) * v0[1]),
                              pack_bf16x2(bf16_lo(xr[kk][1]) * v0[2], bf16_hi(xr[kk][1]) * v0[3]),
                              pack_bf16x2(bf16_lo(xr[kk][2]) * v1[0], bf16_hi(xr[kk][2]) * v1[1]),
                              pack_bf16x2(bf16_lo(xr[kk][3]) * v1[2], bf16_hi(xr[kk][3]) * v1[3])};
#pragma unroll
        for (int u = 0; u < TPW; ++u) acc[u] = mfma32x32x16(bf[kk][u], a, acc[u]);
      }
    }
  };

  for (int k0 = 0; k0 < nsl; k0 += S) {
#pragma unroll
    for (int d = 0; d < S; ++d) {
      const int k = k0 + d;
      lds_barrier();                            // [4] slice k in LDS; slice k - 1 consumed
      if (k < nsl && k % SPC == 0) chunk_start(k / SPC);
      compute(k, d);
    }
  }
  if (var && (pflag & 2)) finish(pseq);        // the last chunk ended a sequence
  if (fin && (nseg > 1 || var)) {
    // a segment's last local state, [b, nseg, H, P * N], each head's in
    // fragment order (hb_off), fp32
    float* dst = fin + ((size_t(b) * nseg + seg) * H + hj) * hstate;
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<f32x4*>(dst + hb_off(pj + l32, 32 * ntile(u) + 8 * jj + 4 * g2, N)) =
            f32x4{acc[u][4 * jj], acc[u][4 * jj + 1], acc[u][4 * jj + 2], acc[u][4 * jj + 3]};
  } else if (fin) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = 32 * ntile(u) + 8 * (r / 4) + 4 * g2 + r % 4;
        fin[(bhj * N + n) * P + pj + l32] = acc[u][r];
      }
    }
  }
}

// The C B^T tiles alone, for segmented launches: their walks take nearly
// every compute unit for the whole launch, so tile work-groups placed behind
// them (as the whole-row launch does) would all run on the few units left.
// The tiles are the ones chunk_scores_tile computes, at the same places.
// The same tiles with the chunk's B rows staged in LDS once (Q x N bf16,
// 128 KB at Q 256, N 256; each 16-byte piece p of row r at piece p ^ (r % 8),
// so the 32 rows a wave reads at one piece fall on different banks): a
// work-group per (batch, chunk, group) of 8 waves, wave w holding the C rows
// of 32-row block w (w < 4) or 11 - w (w >= 4), so the two waves of a SIMD
// hold blocks k and 7 - k (lpc + 1 tiles per SIMD at Q 256); each tile reads
// its B block from LDS. B crosses from memory once per chunk instead of once
// per tile.
template <int N>
__global__ __launch_bounds__(512) void chunk_scores_lds_kernel(const uint16_t* __restrict__ Bm,
                                                               const uint16_t* __restrict__ Cm,
                                                               uint16_t* __restrict__ CB, int T, int G, int Q,
                                                               int nc, const int4* __restrict__ tab,
                                                               uint16_t* __restrict__ CF) {
  constexpr int RP = N / 8;                     // 16-byte pieces per row
  __shared__ __attribute__((aligned(16))) uint16_t sB[kMaxQ * N];
  const int lpc = Q / 32, ntile = lpc * (lpc + 1) / 2;
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int l32 = lane & 31, g2 = lane >> 5;
  const int g = int(blockIdx.x) % G;
  const int c = (int(blockIdx.x) / G) % nc;
  const int b = int(blockIdx.x) / G / nc;
  const ChunkRows cr = chunk_rows(tab, b, c, T, Q);
  if (cr.n <= 0) return;                        // an unused slot: uniform, before the barrier
  // B rows 0 .. Q-1 of the chunk, copied straight into LDS: the wave's 64
  // lanes fill 64 consecutive 16-byte slots, slot (r, q) taking piece
  // q ^ (r % 8) of row r. Rows past the chunk's tokens repeat its last row:
  // every product they enter meets a zero x or a masked weight in chunk_scan
  // (their rows s lie past every valid output row l >= s). All copies are in
  // flight at once; the wait before the barrier covers them.
  static_assert((kMaxQ * RP) % 512 == 0, "whole waves of copies");
  for (int e0 = 0; e0 < Q * RP; e0 += 512) {
    const int e = e0 + tid, r = e / RP, q = e % RP;
    copy_to_lds16(Bm + ((cr.r0 + min(r, cr.n - 1)) * G + g) * size_t(N) + 8 * (q ^ (r & 7)),
                  &sB[size_t(e0 + 64 * wave) * 8]);
  }
  const int i = wave < 4 ? wave : 11 - wave;    // C row block (wave-uniform)
  const bool mine = i < lpc && 32 * i < cr.n;
  u32x4 cf[N / 16];
  if (mine) {
    const int t = 32 * i + l32;
    const uint16_t* crow = Cm + ((cr.r0 + min(t, cr.n - 1)) * G + g) * size_t(N) + 8 * g2;
#pragma unroll
    for (int ks = 0; ks < N / 16; ++ks) cf[ks] = keep_or_zero(t < cr.n, load16(crow + 16 * ks));
  }
  wait_vmcnt<0>();                              // this wave's B copies are in LDS
  __syncthreads();
  if (!mine) return;
  store_c_frags<N>(CF, cf, b, c, g, i, G, Q, nc, lane);   // (after the barrier: no wait for these stores)
  const size_t base = ((size_t(b) * nc + c) * G + g) * ntile;
  for (int j = 0; j <= i; ++j) {
    const int r = 32 * j + l32;                 // this lane's B row
    f32x16 acc = zero16();
#pragma unroll
    for (int ks = 0; ks < N / 16; ++ks) {
      const int p = 2 * ks + g2;                // pieces n = 16 ks + 8 g2 .. + 7
      const u32x4 bf = *reinterpret_cast<const u32x4*>(&sB[r * N + 8 * (p ^ (r & 7))]);
      acc = mfma32x32x16(bf, cf[ks], acc);      // rows s, column l
    }
    u32x4 lo, hi;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      lo[m] = pack_bf16x2(acc[2 * m], acc[2 * m + 1]);
      hi[m] = pack_bf16x2(acc[8 + 2 * m], acc[8 + 2 * m + 1]);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(CB + (base + size_t(i) * (i + 1) / 2 + j) * 1024 + size_t(lane) * 16);
    dst[0] = lo;
    dst[1] = hi;
  }
}

// The same tiles, one wave per tile (chunk_scores_tile), for segmented
// launches with fewer (chunk, group) rows than work-groups fit on the device
// at once: the row form would leave most units idle.
template <int N>
__global__ __launch_bounds__(kChainThreads) void chunk_scores_tiles_kernel(const uint16_t* __restrict__ Bm,
                                                                         const uint16_t* __restrict__ Cm,
                                                                         uint16_t* __restrict__ CB,
                                                                         const int4* __restrict__ tab, int T, int G,
                                                                         int Q, int nc, long ntiles,
                                                                         uint16_t* __restrict__ CF) {
  const long wid = long(blockIdx.x) * kChainWaves + wave_id();
  if (wid < ntiles) chunk_scores_tile<N, false>(Bm, Cm, CB, nullptr, tab, T, G, Q, nc, wid, threadIdx.x & 63, CF);
}

template <int N, int P, int SPC, int ST, bool F32S, bool REV, bool VAR>
hipError_t launch_chain_np(const FwdShape& s, const ChainPlan& pl, const void* x, const void* B, const void* C,
                           const void* dt, const float* A, float* Acs, float* dtq, void* Hs, const float* init,
                           float* fin, uint16_t* CB, uint16_t* CBt, uint16_t* CF, const float* Hst, float* ghp,
                           float* cdec, float* segdec, const VarWalk& vw, hipStream_t st, const StageEv& ev) {
  constexpr int CW = chain_cols(N, P, SPC, F32S || REV), NW = chain_waves(CW);
  // whole work-groups per row, and the heads of one in one B/C group
  if ((long(s.H) * P) % CW != 0 || (P < CW && (s.H / s.G) % (CW / P) != 0)) return hipErrorInvalidValue;
  const int lpc = s.Q / 32;
  const long alltiles = REV ? 0 : long(s.b) * s.nc * s.G * (lpc * (lpc + 1) / 2);
  const long nchain = long(s.b) * s.H * P / CW * pl.nseg;
  // segmented (packed rows always): the tiles in a launch of their own, cdec
  // and segdec written
  const bool segd = pl.nseg > 1 || pl.var;
  // segmented: the tiles first, as a launch of their own (the stage's start
  // event on it, the stop event on the walk)
  if (alltiles > 0 && !F32S && !CF) return hipErrorInvalidValue;   // the forward's tiles also write C in operand order
  if (segd && alltiles > 0) {
    const long rows = long(s.b) * s.nc * s.G;
    const int4* tab = pl.var ? vw.tab : nullptr;
    if (rows >= 2L * device_units()) {
      hipExtLaunchKernelGGL((chunk_scores_lds_kernel<N>), dim3(unsigned(rows)), dim3(512), 0, st, ev.start, nullptr,
                            0, static_cast<const uint16_t*>(B), static_cast<const uint16_t*>(C), CB, s.T, s.G, s.Q,
                            s.nc, tab, CF);
    } else {
      hipExtLaunchKernelGGL((chunk_scores_tiles_kernel<N>), dim3(unsigned((alltiles + kChainWaves - 1) / kChainWaves)),
                            dim3(kChainThreads), 0, st, ev.start, nullptr, 0, static_cast<const uint16_t*>(B),
                            static_cast<const uint16_t*>(C), CB, tab, s.T, s.G, s.Q, s.nc, alltiles, CF);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long ntiles = segd ? 0 : alltiles;
  const long blocks = nchain + (ntiles + NW - 1) / NW;
  hipExtLaunchKernelGGL((chunk_state_chain_kernel<N, P, SPC, ST, F32S, REV, VAR>), dim3(unsigned(blocks)),
                        dim3(64 * NW), 0, st, segd && alltiles > 0 ? nullptr : ev.start, ev.stop, 0,
                        static_cast<const uint16_t*>(x),
                        static_cast<const uint16_t*>(B), static_cast<const uint16_t*>(dt), A, Acs, dtq, Hs, init, fin,
                        static_cast<const uint16_t*>(C), CB, CBt, Hst, ghp, segd ? cdec : nullptr,
                        segd ? segdec : nullptr, s.T, s.H, s.G, s.Q, s.nc, s.b, pl.nseg, pl.seglen, int(nchain),
                        ntiles, VAR ? vw : VarWalk{}, segd ? nullptr : CF);
  return hipGetLastError();
}

template <int N, int P, int MODE>
hipError_t launch_np(const FwdShape& s, const void* x, const void* B, const void* C, const void* dt,
                     const float* A, float* Acs, float* dtq, float* S, uint16_t* CB, uint16_t* CBt, uint16_t* CF,
                     const int4* tab, hipStream_t st, const StageEv& ev) {
  const int lpc = s.Q / 32;
  const long ntiles = MODE == 2 ? 0 : long(s.b) * s.nc * s.G * (lpc * (lpc + 1) / 2);
  // score work-groups first (they start with the first wave of work-groups),
  // padded to a multiple of 8 so the chunk-state work-groups keep their XCD
  const long nscore = ((ntiles + kWaves - 1) / kWaves + 7) / 8 * 8;
  const long blocks = nscore + long(s.b) * s.nc * s.H;
  hipExtLaunchKernelGGL((chunk_state_mfma_kernel<N, P, MODE>), dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                        ev.start, ev.stop, 0, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(B),
                        static_cast<const uint16_t*>(dt), A, Acs, dtq, S, static_cast<const uint16_t*>(C), CB,
                        CBt, tab, s.T, s.H, s.G, s.Q, s.nc, int(nscore), ntiles, CF);
  return hipGetLastError();
}

template <int N, int MODE>
hipError_t launch_n(const FwdShape& s, const void* x, const void* B, const void* C, const void* dt,
                    const float* A, float* Acs, float* dtq, float* S, uint16_t* CB, uint16_t* CBt, uint16_t* CF,
                    const int4* tab, hipStream_t st, const StageEv& ev) {
  switch (s.P) {
    case 32: return launch_np<N, 32, MODE>(s, x, B, C, dt, A, Acs, dtq, S, CB, CBt, CF, tab, st, ev);
    case 64: return launch_np<N, 64, MODE>(s, x, B, C, dt, A, Acs, dtq, S, CB, CBt, CF, tab, st, ev);
    case 128: return launch_np<N, 128, MODE>(s, x, B, C, dt, A, Acs, dtq, S, CB, CBt, CF, tab, st, ev);
  }
  return hipErrorInvalidValue;
}

template <int MODE>
hipError_t launch_mode(const FwdShape& s, const void* x, const void* B, const void* C, const void* dt,
                       const float* A, float* Acs, float* dtq, float* S, uint16_t* CB, uint16_t* CBt,
                       uint16_t* CF, const int4* tab, hipStream_t st, const StageEv& ev) {
  switch (s.N) {
    case 32: return launch_n<32, MODE>(s, x, B, C, dt, A, Acs, dtq, S, CB, CBt, CF, tab, st, ev);
    case 64: return launch_n<64, MODE>(s, x, B, C, dt, A, Acs, dtq, S, CB, CBt, CF, tab, st, ev);
    case 128: return launch_n<128, MODE>(s, x, B, C, dt, A, Acs, dtq, S, CB, CBt, CF, tab, st, ev);
    case 256: return launch_n<256, MODE>(s, x, B, C, dt, A, Acs, dtq, S, CB, CBt, CF, tab, st, ev);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_state_mfma(const FwdShape& s, const void* x, const void* B, const void* C,
                                   const void* dt, const float* A, float* Acs, float* dtq,
                                   float* S, uint16_t* CB, uint16_t* CF, const int4* tab, hipStream_t st,
                                   const StageEv& ev) {
  if (!CF) return hipErrorInvalidValue;
  return launch_mode<0>(s, x, B, C, dt, A, Acs, dtq, S, CB, nullptr, CF, tab, st, ev);
}

template <int N_, int P_>
struct ChainNP {
  static constexpr int n = N_, p = P_;
};

// Compute units of the current device, read once per device.
int device_units() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
  if (dev < kMaxDevices) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// The fused launch pays off when its work-groups (one per batch row, 64
// columns and segment) fill the chip in one round: each is a serial walk
// over its slices, so fewer than half the compute units leave too many
// idle, and more than fit at once (one per unit with five slices resident;
// at dstate 128 two per unit with three) run in two rounds of the whole
// walk; such shapes take the two-kernel path. Headdim 32 pairs two heads,
// which must share a B/C group. Where whole rows give fewer walks than half
// the units (few, long rows), the forward cuts each row into segments of
// equal chunk counts (the last may be shorter), as many as one walk per unit
// allows and at most one per chunk; if that still leaves more than half the
// units idle, the two-kernel path runs.
namespace {
// the shapes the walk serves: dstate 128 or 256, headdim 32, 64 or 128,
// chunks of whole 64-token slices, and where a work-group of cw columns
// holds several heads (cw / P), whole groups of them in one B/C group
bool chain_shape_ok(const FwdShape& s, int cw) {
  if (!((s.N == 128 || s.N == 256) && (s.P == 32 || s.P == 64 || s.P == 128) && s.Q % kChainSK == 0)) return false;
  return !(s.P < cw && (s.H / s.G) % (cw / s.P) != 0);
}
// walks that fit a unit at once: two at dstate 128 with a chunk start at
// most every other slice (the registers of a chunk start every slice do not
// fit that occupancy), else one
long chain_per_unit(const FwdShape& s) { return s.N == 128 && s.Q >= 2 * kChainSK ? 2 : 1; }
}  // namespace

ChainPlan chunk_state_chain_plan_for(const FwdShape& s, int cus, bool allow_segments) {
  ChainPlan pl;
  // the forward's walks (segments allowed) at their column width, the
  // backward's (whole rows) at 64
  const int cw = chain_cols(s.N, s.P, s.Q / kChainSK, !allow_segments);
  if (!chain_shape_ok(s, cw)) return pl;
  if (cus <= 0 || s.nc < 1) return pl;
  const long wgs = long(s.b) * s.H * s.P / cw;
  const long per_unit = chain_per_unit(s);
  if (wgs > per_unit * cus) return pl;
  if (2 * wgs >= cus) {
    pl.ok = true;
    pl.nseg = 1;
    pl.seglen = s.nc;                      // one segment: the whole row
    pl.two = wgs > cus;
    return pl;
  }
  if (!allow_segments) return pl;
  // segments: one walk per unit
  const int want = int(std::min<long>(s.nc, cus / wgs));
  const int seglen = (s.nc + want - 1) / want;
  const int nseg = (s.nc + seglen - 1) / seglen;
  if (2 * wgs * nseg < cus) return pl;   // too little work to fill half the chip
  pl.ok = true;
  pl.nseg = nseg;
  pl.seglen = seglen;
  return pl;
}

// Packed sequences: the row of chunk slots is cut like a batch row into
// equal segments, as many as fill the device with walks in one round (two
// per unit where they fit) and at most one per slot; sequences begin and end
// anywhere inside a segment. Any number of sequences is served.
ChainPlan varlen_chain_plan_for(const FwdShape& s, int nseq, int cus) {
  ChainPlan pl;
  const int cw = chain_cols(s.N, s.P, s.Q / kChainSK, false);
  if (!chain_shape_ok(s, cw) || s.b != 1 || cus <= 0 || nseq < 1 || s.nc < 1) return pl;
  const long cpr = long(s.H) * s.P / cw;
  const long per_unit = chain_per_unit(s);
  const long want = std::min<long>(s.nc, per_unit * cus / cpr);
  if (want < 1) return pl;                 // not even one segment per column block fits at once
  // at most kVarWalkSlots slots per segment (their table entries sit in LDS):
  // longer rows take more segments than fit at once
  pl.seglen = int(std::min<long>((s.nc + want - 1) / want, kVarWalkSlots));
  pl.nseg = (s.nc + pl.seglen - 1) / pl.seglen;
  pl.ok = true;
  pl.var = true;
  pl.two = per_unit == 2 && long(pl.nseg) * cpr > cus;
  return pl;
}

ChainPlan chunk_state_chain_plan(const FwdShape& s, bool allow_segments) {
  return chunk_state_chain_plan_for(s, device_units(), allow_segments);
}

bool chain_plan_valid(const FwdShape& s, const ChainPlan& pl) {
  return pl.ok && pl.nseg >= 1 && pl.seglen >= 1 && long(pl.nseg - 1) * pl.seglen < s.nc &&
         long(pl.nseg) * pl.seglen >= s.nc;
}

bool chunk_state_chain_ok(const FwdShape& s) { return chunk_state_chain_plan(s, false).ok; }

template <bool F32S, bool REV>
hipError_t launch_chain(const FwdShape& s, const ChainPlan& pl, const void* x, const void* B, const void* C,
                        const void* dt, const float* A, float* Acs, float* dtq, void* Hs, const float* init,
                        float* fin, uint16_t* CB, uint16_t* CBt, uint16_t* CF, const float* Hst, float* ghp,
                        float* cdec, float* segdec, hipStream_t st, const StageEv& ev, const VarWalk& vw = VarWalk{}) {
  // every walk must own at least one chunk and the segments must cover the
  // row exactly: a walk without slices would clamp its copies to slice -1
  const bool ok = chain_plan_valid(s, pl) &&
                  (pl.var ? s.b == 1 && vw.tab && vw.nseq >= 1 && cdec && segdec && fin && !F32S && !REV &&
                                pl.seglen <= kVarWalkSlots
                          : !((F32S || REV) && pl.nseg != 1));
  if (!ok) return hipErrorInvalidValue;
  auto by_q = [&](auto np) -> hipError_t {
    using NP = decltype(np);
    constexpr int S1 = NP::n == 128 ? 5 : 3;
    // one instantiation per (slices per chunk, slices resident); the walk
    // over packed rows is an instantiation of its own
    auto go = [&](auto spc, auto stg) -> hipError_t {
      constexpr int SPC_ = decltype(spc)::value, ST_ = decltype(stg)::value;
      if constexpr (!F32S && !REV) {
        if (pl.var)
          return launch_chain_np<NP::n, NP::p, SPC_, ST_, false, false, true>(
              s, pl, x, B, C, dt, A, Acs, dtq, Hs, init, fin, CB, CBt, CF, Hst, ghp, cdec, segdec, vw, st, ev);
      }
      return launch_chain_np<NP::n, NP::p, SPC_, ST_, F32S, REV, false>(
          s, pl, x, B, C, dt, A, Acs, dtq, Hs, init, fin, CB, CBt, CF, Hst, ghp, cdec, segdec, vw, st, ev);
    };
    if (pl.two && NP::n == 128) {
      // two work-groups per unit (three slices resident; chunks of two or
      // four slices, which the plan ensures) where one per unit would not
      // hold them all
      if constexpr (REV) {
        return hipErrorInvalidValue;            // one per unit only (registers)
      } else {
        switch (s.Q / kChainSK) {
          case 2: return go(IntC<2>{}, IntC<3>{});
          case 4: return go(IntC<4>{}, IntC<3>{});
        }
        return hipErrorInvalidValue;
      }
    }
    switch (s.Q / kChainSK) {
      case 1: return go(IntC<1>{}, IntC<S1>{});
      case 2: return go(IntC<2>{}, IntC<S1>{});
      case 4: return go(IntC<4>{}, IntC<S1>{});
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

hipError_t launch_chunk_state_chain(const FwdShape& s, const ChainPlan& pl, const void* x, const void* B,
                                    const void* C, const void* dt, const float* A, float* Acs, float* dtq,
                                    uint16_t* Hb, const float* init, float* fin, uint16_t* CB, uint16_t* CF,
                                    float* cdec, float* segdec, hipStream_t st, const StageEv& ev) {
  if (pl.var) return hipErrorInvalidValue;
  return launch_chain<false, false>(s, pl, x, B, C, dt, A, Acs, dtq, Hb, init, fin, CB, nullptr, CF, nullptr,
                                    nullptr, cdec, segdec, st, ev);
}

hipError_t launch_chunk_state_chain_varlen(const FwdShape& s, const ChainPlan& pl, const void* x, const void* B,
                                           const void* C, const void* dt, const float* A, float* Acs, float* dtq,
                                           uint16_t* Hb, const float* init, float* segS, uint16_t* CB,
                                           uint16_t* CF, float* cdec, float* segdec, const VarWalk& vw,
                                           hipStream_t st, const StageEv& ev) {
  if (!pl.var) return hipErrorInvalidValue;
  return launch_chain<false, false>(s, pl, x, B, C, dt, A, Acs, dtq, Hb, init, segS, CB, nullptr, CF, nullptr,
                                    nullptr, cdec, segdec, st, ev, vw);
}

hipError_t launch_chunk_state_chain_bwd(const FwdShape& s, const void* x, const void* B, const void* C,
                                        const void* dt, const float* A, float* Acs, float* dtq, float* Hst,
                                        const float* init, float* fin, uint16_t* CBf, uint16_t* CBt,
                                        hipStream_t st) {
  return launch_chain<true, false>(s, chunk_state_chain_plan(s, false), x, B, C, dt, A, Acs, dtq, Hst, init, fin,
                                   CBf, CBt, nullptr, nullptr, nullptr, nullptr, nullptr, st, StageEv{});
}

// The reverse walk holds a run of H_c per lane besides the accumulators, which
// the two-per-unit occupancy leaves no room for: one work-group per unit.
bool chunk_grad_chain_ok(const FwdShape& s) {
  const ChainPlan pl = chunk_state_chain_plan(s, false);
  return pl.ok && !pl.two;
}

hipError_t launch_chunk_grad_chain_bwd(const FwdShape& s, const void* dy, const void* C, const void* dt,
                                       const float* A, const float* dfinal, uint16_t* Gb, float* dinit,
                                       const float* Hst, float* ghp, hipStream_t st) {
  if (!chunk_grad_chain_ok(s)) return hipErrorInvalidValue;
  return launch_chain<false, true>(s, chunk_state_chain_plan(s, false), dy, C, nullptr, dt, A, nullptr, nullptr, Gb,
                                   dfinal, dinit, nullptr, nullptr, nullptr, Hst, ghp, nullptr, nullptr, st,
                                   StageEv{});
}

hipError_t launch_chunk_state_mfma_bwd(const FwdShape& s, const void* x, const void* B, const void* C,
                                       const void* dt, const float* A, float* Acs, float* dtq, float* S,
                                       uint16_t* CB, uint16_t* CBt, hipStream_t st) {
  return launch_mode<1>(s, x, B, C, dt, A, Acs, dtq, S, CB, CBt, nullptr, nullptr, st, StageEv{});
}

hipError_t launch_chunk_dstates_mfma(const FwdShape& s, const void* dy, const void* C, const void* dt,
                                     const float* A, float* dS, hipStream_t st) {
  return launch_mode<2>(s, dy, C, nullptr, dt, A, nullptr, nullptr, dS, nullptr, nullptr, nullptr, nullptr, st,
                        StageEv{});
}

}  // namespace ssd
