// ssd_internal.h -- private declarations shared by the HIP translation units of
// libssd.so (device helpers, problem shape, workspace layout, launchers).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ssd_api.h"

namespace ssd {

// Native clang vector types (usable with the nontemporal builtins, unlike the
// HIP_vector_type structs).
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Element access. bf16 values travel as their raw 16-bit patterns (uint16_t);
// the arithmetic is always fp32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// fp32 -> bf16, round to nearest, ties to even (NaN stays NaN): the gfx950
// conversion instruction (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

// two fp32 -> packed bf16 pair (lo in bits 0..15), one conversion instruction
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{lo, hi}, b2));
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) { return f32_to_bf16(v); }

// Index of this wave inside its work-group, as a wave-uniform (scalar) value:
// threadIdx.x / 64 is the same on every lane of a wave, but the compiler only
// treats it as uniform -- and branches on it as scalar branches instead of
// executing both sides under an exec mask -- when it comes from readfirstlane.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
}

// exp(x) through the hardware base-2 exponential: exp(x) = 2^(x * log2(e)).
__device__ __forceinline__ float exp_fast(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// ---------------------------------------------------------------------------
// Chunks of a forward call. Every kernel sees a chunk as its first token
// row in the token-major tensors (row = b * T + t) and its number of valid
// tokens; tokens past them count as dt = 0 (nothing enters the state). For
// a batch of equal-length rows both follow from (b, c).
//
// Packed variable-length sequences (one row of T tokens, sequence i being
// tokens cu[i] .. cu[i+1]-1) are cut into chunks that each lie inside one
// sequence; chunk k of sequence i takes slot floor(cu[i] / Q) + i + k. The
// slots of one sequence are consecutive, later sequences take later slots
// (a chunk of sequence i starts before sequence i+1 does, and i grows by
// one), and the last slot is below ceil(T / Q) + nseq. A table gives each
// slot tab[c] = {first row, valid tokens (0: unused slot), sequence, flags
// (bit 0: first chunk of its sequence, bit 1: last)}.
// ---------------------------------------------------------------------------
struct ChunkRows {
  long r0;   // first token row
  int n;     // valid tokens (0 .. Q)
};

__host__ __device__ __forceinline__ int clamp_int(int v, int lo, int hi) { return v < lo ? lo : v > hi ? hi : v; }

// rows stay inside [0, T) whatever a table entry holds: the first row in
// [0, T], at most T - r0 valid tokens (0 or less: no rows)
__device__ __forceinline__ ChunkRows chunk_rows(const int4* tab, int b, int c, int T, int Q) {
  if (tab) {
    const int4 e = tab[c];
    const int r0 = clamp_int(e.x, 0, T);
    return ChunkRows{long(r0), min(e.y, T - r0)};
  }
  return ChunkRows{long(b) * T + long(c) * Q, min(Q, T - c * Q)};
}

// The token span of sequence i: offsets are clamped into [0, T] and a span
// never ends before it starts, so any offsets give in-bounds spans.
// Well-formed offsets (0 = cu[0] <= ... <= cu[nseq] = T) are used as given.
__host__ __device__ __forceinline__ void varlen_span(const int* cu, int i, int T, int& s0, int& len) {
  s0 = clamp_int(cu[i], 0, T);
  const int s1 = clamp_int(cu[i + 1], s0, T);
  len = s1 - s0;
}

// first chunk slot of sequence i, which starts at token s0
__host__ __device__ __forceinline__ int varlen_first_slot(int s0, int i, int Q) { return s0 / Q + i; }

// chunk slots for T tokens in nseq sequences
__host__ __device__ __forceinline__ int varlen_slots(int T, int nseq, int Q) { return (T + Q - 1) / Q + nseq; }

// The table entry of chunk slot c, built slot by slot (the table kernel, one
// thread per slot): the sequence holding c is the last one whose first slot
// is <= c (first(i) = floor(s0_i / Q) + i grows with i for well-formed
// offsets, and a sequence's chunks end before the next sequence's first
// slot), found by bisection over first(); `first` gives first(i) for
// 0 <= i < nseq. Slot c holds chunk c - first(i) of that sequence when the
// sequence reaches that far, else nothing. For well-formed offsets every
// sequence's chunks fill consecutive slots from its first and the slots
// between sequences stay empty; for any offsets an entry is one chunk of a
// clamped span or empty, so every row it names lies inside the tokens.
template <class First>
__host__ __device__ inline int4 varlen_slot_entry(const int* cu, int nseq, int T, int Q, int c, First first) {
  int lo = 0, hi = nseq - 1, i = -1;
  while (lo <= hi) {
    const int mid = (lo + hi) >> 1;
    if (first(mid) <= c) {
      i = mid;
      lo = mid + 1;
    } else {
      hi = mid - 1;
    }
  }
  if (i < 0) return int4{0, 0, 0, 0};
  int s0, len;
  varlen_span(cu, i, T, s0, len);
  const int nch = (len + Q - 1) / Q;
  const int k = c - varlen_first_slot(s0, i, Q);
  if (k < 0 || k >= nch) return int4{0, 0, 0, 0};
  const int flags = (k == 0 ? 1 : 0) | (k == nch - 1 ? 2 : 0);
  return int4{s0 + k * Q, len - k * Q < Q ? len - k * Q : Q, i, flags};
}

// ---------------------------------------------------------------------------
// Problem shape of one forward call.
// ---------------------------------------------------------------------------
struct FwdShape {
  int b, T, H, P, N, G, Q, nc;  // batch, tokens, heads, headdim, dstate, groups, chunk, chunks
};

// Which kernels a forward call uses. The bf16 MFMA kernels cover dstate and
// headdim that are multiples of 32 (dstate in {32, 64, 128, 256}, headdim in
// {32, 64, 128}) and chunk_len >= 32; every other shape and the fp32 path run
// the generic fp32-FMA kernels.
inline bool use_mfma_path(const FwdShape& s, ssd_dtype t) {
  const bool n_ok = s.N == 32 || s.N == 64 || s.N == 128 || s.N == 256;
  const bool p_ok = s.P == 32 || s.P == 64 || s.P == 128;
  return t == SSD_BF16 && n_ok && p_ok && s.Q >= 32;
}

// How the bf16 matrix-core forward computes the states entering each chunk
// (chunk_state_mfma.hip): ok = the fused chunk-state + state-passing walk
// (else a chunk_state and a state_passing launch); nseg segments of seglen
// chunks per batch row (1: whole rows); two = two walks per compute unit.
struct ChainPlan {
  bool ok = false;
  int nseg = 1, seglen = 0;
  bool two = false;
  // packed sequences: the row of chunk slots cut into nseg segments of
  // seglen slots, the walks reset at sequence starts (always segmented,
  // whatever nseg)
  bool var = false;
};
// allow_segments = false: whole rows only (the backward's walks). The plan
// for a device with `cus` compute units, and for the current device.
ChainPlan chunk_state_chain_plan_for(const FwdShape& s, int cus, bool allow_segments);
ChainPlan chunk_state_chain_plan(const FwdShape& s, bool allow_segments);
// pl.ok and its segments cover the row's chunks exactly, each at least one
bool chain_plan_valid(const FwdShape& s, const ChainPlan& pl);
// Packed sequences (s: batch 1, T packed tokens, nc chunk slots) through the
// fused walk: the slot row cut into equal segments, as many as fill the
// device with walks (one per segment and 64 columns) in one round; ok =
// false where the walk does not serve the shape (the per-chunk path runs).
ChainPlan varlen_chain_plan_for(const FwdShape& s, int nseq, int cus);
// compute units of the current device (read once per device; 0 without one)
constexpr int kMaxDevices = 64;
int device_units();

// Layout of one head's bf16 state entering a chunk (the matrix-core path's
// Hb, P x N per (batch, chunk, head)): matrix-core fragment order. Element
// (p, n) sits at
//   ((((p / 32) * (N / 32) + n / 32) * 4 + (n % 32) / 8) * 64
//       + p % 32 + 32 * ((n % 8) / 4)) * 4 + n % 4,
// i.e. runs of four consecutive n; each 32 x 32 block (p / 32, n / 32) is
// 1024 consecutive elements, four groups of 64 runs. It is the order in
// which the fused walk holds a state in its MFMA accumulators (lane
// p % 32 + 32 ((n % 8) / 4), register 4 ((n % 32) / 8) + n % 4), so each
// of its stores writes 512 contiguous bytes. Needs P and N multiples of 32.
__host__ __device__ __forceinline__ size_t hb_off(int p, int n, int N) {
  return ((size_t((p >> 5) * (N >> 5) + (n >> 5)) * 4 + ((n & 31) >> 3)) * 64 + (p & 31) + 32 * ((n & 7) >> 2)) * 4 +
         (n & 3);
}

// Workspace layout (byte offsets, each 256-byte aligned):
//   acs [b, H, nc, Q] f32    cumulative dt*A inside each chunk (inclusive)
//   dtq [b, H, nc, Q] f32    dt widened to fp32, 0 past the end of the sequence
//   st  [b, nc, H, P, N] f32 chunk states, stored transposed (n fastest); on
//                            the generic path overwritten in place by the
//                            states entering each chunk. Absent on the fused
//                            path, except with segments: [b, nseg, H, P * N]
//                            (fragment order), each segment's last local
//                            state, then (in place) the state entering each
//                            segment
//   hb  [b, nc, H, P * N] bf16 states entering each chunk, each head's in
//                            fragment order (hb_off; MFMA path only; with
//                            segments, the local ones)
//   cb  [b, nc, G, ntile, 64, 16] bf16 C B^T tiles of each chunk (MFMA path
//       only; ntile = lpc (lpc + 1) / 2 lower-triangle tiles, lpc = Q / 32)
//   cf  [b, nc, G, Q / 32, N / 16, 64, 8] bf16 (MFMA path only): C in the
//       order chunk_scan's matrix-core operands take it (store_c_frags in
//       chunk_state_mfma.hip), written with the C B^T tiles
//   cdec [b, H, nc] f32, segdec [b, H, nseg] f32 (segments only): summed
//       chunk decay exponents from the segment's start to each chunk, and over
//       each segment
struct WsLayout {
  size_t acs, dtq, st, hb, cb, cf, cdec, segdec, total;
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline WsLayout ws_layout(const FwdShape& s, bool mfma, const ChainPlan& pl) {
  WsLayout w;
  const size_t row = size_t(s.b) * s.H * s.nc * s.Q * sizeof(float);
  const size_t nst = size_t(s.b) * s.nc * s.H * s.N * s.P;
  const bool fused = mfma && pl.ok;
  const bool seg = fused && (pl.nseg > 1 || pl.var);
  const size_t nstf = !fused ? nst : seg ? size_t(s.b) * pl.nseg * s.H * s.N * s.P : 0;
  w.acs = 0;
  w.dtq = align_up(w.acs + row, 256);
  w.st = align_up(w.dtq + row, 256);
  w.hb = align_up(w.st + nstf * sizeof(float), 256);
  if (!mfma) {
    w.cb = w.cf = w.cdec = w.segdec = w.total = w.hb;
    return w;
  }
  w.cb = align_up(w.hb + nst * sizeof(uint16_t), 256);
  const size_t lpc = size_t(s.Q) / 32, ntile = lpc * (lpc + 1) / 2;
  w.cf = align_up(w.cb + size_t(s.b) * s.nc * s.G * ntile * 1024 * sizeof(uint16_t), 256);
  w.cdec = align_up(w.cf + size_t(s.b) * s.nc * s.G * s.Q * s.N * sizeof(uint16_t), 256);
  w.segdec = align_up(w.cdec + (seg ? size_t(s.b) * s.H * s.nc * sizeof(float) : 0), 256);
  w.total = align_up(w.segdec + (seg ? size_t(s.b) * s.H * pl.nseg * sizeof(float) : 0), 256);
  return w;
}

// XCD-aware block order: the hardware hands consecutive work-groups to the 8
// XCDs round-robin, so block id k runs on XCD k % 8. Renumbering blocks so that
// each XCD receives one contiguous range of logical ids keeps logical
// neighbours (which share B/C rows) inside one XCD's L2. XCD x holds
// ceil((nblocks - x) / 8) blocks: q + 1 for the first r = nblocks % 8 of them,
// q = nblocks / 8 for the rest, so its range starts at x q + min(x, r); a
// bijection of [0, nblocks) for any nblocks.
__host__ __device__ __forceinline__ int xcd_swizzle(int bid, int nblocks) {
  const int q = nblocks / 8, r = nblocks % 8, x = bid % 8;
  return x * q + (x < r ? x : r) + bid / 8;
}

// Optional start / stop events of one forward launch. The launchers pass them
// to hipExtLaunchKernel, which records them as part of the kernel's own
// dispatch, so the pair brackets exactly that kernel's execution (null: no
// events).
struct StageEv {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// ---------------------------------------------------------------------------
// Launchers (one translation unit each). All return the launch status.
// ---------------------------------------------------------------------------
hipError_t launch_chunk_cumsum(const FwdShape& s, ssd_dtype dt_type, const void* dt, const float* A,
                               float* Acs, float* dtq, hipStream_t st, const StageEv& ev = StageEv{});

// S: chunk states [b, nc, H, P, N] f32 (generic path: from Acs / dtq that
// chunk_cumsum wrote).
hipError_t launch_chunk_state(const FwdShape& s, ssd_dtype type, const void* x, const void* B,
                              const float* Acs, const float* dtq, float* S, hipStream_t st, const StageEv& ev = StageEv{});
// Matrix-core path: S^T [b, nc, H, P, N] f32; the same launch also computes
// the in-chunk cumulative sums (written to Acs / dtq) and the C B^T tiles
// (CB [b, nc, G, ntile, 64, 16] bf16) with C in chunk_scan's operand order
// (CF, the workspace's cf region) for the kernels after it.
// tab: the chunk table of packed variable-length sequences, or nullptr.
hipError_t launch_chunk_state_mfma(const FwdShape& s, const void* x, const void* B, const void* C,
                                   const void* dt, const float* A, float* Acs, float* dtq,
                                   float* S, uint16_t* CB, uint16_t* CF, const int4* tab, hipStream_t st,
                                   const StageEv& ev = StageEv{});

// Chunk states and state passing fused (equal-length rows, bf16 MFMA path):
// writes Acs, dtq, the C B^T tiles and Hb (states entering each chunk, bf16)
// and final (fp32, may be null), without the fp32 chunk states. Only for the
// shapes chunk_state_chain_plan accepts (enough (batch row, 64-column,
// segment) walks to fill the chip in one round; dstate 128 or 256;
// chunk_len a multiple of 64). With segments (pl.nseg > 1), Hb holds the
// local states, fin receives each segment's last local state
// ([b, nseg, H, P, N] fp32) and cdec / segdec the summed decay exponents.
bool chunk_state_chain_ok(const FwdShape& s);   // whole rows
hipError_t launch_chunk_state_chain(const FwdShape& s, const ChainPlan& pl, const void* x, const void* B,
                                    const void* C, const void* dt, const float* A, float* Acs, float* dtq,
                                    uint16_t* Hb, const float* init, float* fin, uint16_t* CB, uint16_t* CF,
                                    float* cdec, float* segdec, hipStream_t st, const StageEv& ev = StageEv{});
// Packed sequences (pl from varlen_chain_plan_for; s: batch 1, nc chunk
// slots): the slot row cut into pl.nseg equal segments, one walk per
// (segment, 64 columns), rows and sequence starts / ends from the chunk table.
// A walk starts from zero and restarts from a sequence's initial state (init
// [nseq, H, N, P], may be null) at each chunk that begins a sequence; cdec
// and segdec are -inf from the first restart on, so that only the chunks of
// the sequence the segment continues take the state entering the segment.
// A sequence that begins and ends inside one walk gets its final state
// (fin [nseq, H, N, P], may be null) from that walk; where the segment's
// first sequence continues from before and ends inside it, the walk leaves
// its local end state in F ([nseg, H, P * N] fp32, fragment order), its
// summed decay exponent from the segment's start in fdec [H, nseg] and the
// sequence in fseq[seg] (else -1), for the recurrence over segments. segS
// receives each segment's last local state as for segmented batch rows.
struct VarWalk {
  const int4* tab = nullptr;
  int nseq = 0;
  float* fin = nullptr;
  float* F = nullptr;
  float* fdec = nullptr;
  int* fseq = nullptr;
};
hipError_t launch_chunk_state_chain_varlen(const FwdShape& s, const ChainPlan& pl, const void* x, const void* B,
                                           const void* C, const void* dt, const float* A, float* Acs, float* dtq,
                                           uint16_t* Hb, const float* init, float* segS, uint16_t* CB,
                                           uint16_t* CF, float* cdec, float* segdec, const VarWalk& vw,
                                           hipStream_t st, const StageEv& ev = StageEv{});
// The same for the backward's recomputation: the states entering each chunk
// as fp32 in Hst ([b, c, h, p, n], what state_passing leaves over the chunk
// states) and the C B^T tiles as fp32 in both orientations (CBf, CBt, as
// launch_chunk_state_mfma_bwd writes them).
hipError_t launch_chunk_state_chain_bwd(const FwdShape& s, const void* x, const void* B, const void* C,
                                        const void* dt, const float* A, float* Acs, float* dtq, float* Hst,
                                        const float* init, float* fin, uint16_t* CBf, uint16_t* CBt,
                                        hipStream_t st);
// The backward's reverse pass through the same walk in reverse (shapes
// chunk_state_chain_ok accepts): the gradients G_c of the states leaving each
// chunk as bf16 in Gb ([b, c, h, p, n]), their dot products with Hst (the
// fp32 states entering each chunk) in P / 16 partials per (b, h, c) in ghp,
// and d init (fp32 [b, h, n, p], may be null), from dy, C and dfinal (may
// be null).
bool chunk_grad_chain_ok(const FwdShape& s);   // one work-group per compute unit
hipError_t launch_chunk_grad_chain_bwd(const FwdShape& s, const void* dy, const void* C, const void* dt,
                                       const float* A, const float* dfinal, uint16_t* Gb, float* dinit,
                                       const float* Hst, float* ghp, hipStream_t st);

// Hb == nullptr: states entering each chunk overwrite S in place (fp32);
// otherwise they are written to Hb as bf16 (fragment order, hb_off) and S is
// left as it was. sfrag: each head's S is in fragment order (the segment
// states of the fused walk) instead of [p][n] rows.
hipError_t launch_state_passing(const FwdShape& s, float* S, uint16_t* Hb, const float* Acs,
                                const float* init, float* final_state, hipStream_t st, const StageEv& ev = StageEv{},
                                bool sfrag = false);

// Packed variable-length sequences (batch 1, chunk slots as above, matrix-core
// path): one recurrence per sequence over its own slots; init / final_state
// are [nseq, H, N, P] (a sequence without tokens: final = init, or zero).
hipError_t launch_state_passing_varlen(const FwdShape& s, const float* S, uint16_t* Hb, const float* Acs,
                                       const int* cu, int nseq, const float* init, float* final_state,
                                       hipStream_t st, const StageEv& ev = StageEv{});
// The recurrence over the packed walks' segments (s.nc = nseg segments):
// carry_0 = 0; for each segment k in order, the state entering it is
// carry_k (written over S[k], which held its last local state E_k), the
// final state of fseq[k] (if >= 0) is F_k + exp(fdec_k) carry_k, and
// carry_{k+1} = exp(segdec_k) carry_k + E_k (segdec_k = -inf where a
// sequence began inside segment k). A sequence without tokens gets its
// initial state (or zero) as its final state. final_state may be null.
hipError_t launch_varlen_segment_recurrence(const FwdShape& s, float* S, const float* F, const float* segdec,
                                            const float* fdec, const int* fseq, const int* cu, int nseq,
                                            const float* init, float* final_state, hipStream_t st,
                                            const StageEv& ev = StageEv{});

// Generic path reads Hst (fp32, [b, nc, H, P, N]) and C; MFMA path reads Hb
// (bf16), the C B^T tiles CB and C in operand order (Cf).
hipError_t launch_chunk_scan(const FwdShape& s, ssd_dtype type, bool mfma, const void* x,
                             const void* B, const void* C, const float* Acs, const float* dtq,
                             const float* Hst, const uint16_t* Hb, const uint16_t* CB, const uint16_t* Cf,
                             const float* D, void* y, hipStream_t st, const StageEv& ev = StageEv{});
// Segmented states (ChainPlan::nseg > 1): the state entering chunk c of
// segment k >= 1 is Hb_c + exp(cdec_c) Hin_k, Hin [b, nseg, H, P * N] fp32,
// each head's in fragment order (hb_off). var: packed sequences (rows from
// the chunk table; dstate 128 or 256), segments of seglen slots, cdec -inf
// for the chunks that take no correction.
struct SegStates {
  const float* Hin = nullptr;
  const float* cdec = nullptr;
  int nseg = 1, seglen = 0;
  bool var = false;
};
hipError_t launch_chunk_scan_mfma(const FwdShape& s, const void* x, const uint16_t* CB,
                                  const uint16_t* Cf, const float* Acs, const float* dtq,
                                  const uint16_t* Hb, const float* D, void* y, const int4* tab,
                                  hipStream_t st, const StageEv& ev = StageEv{},
                                  const SegStates& seg = SegStates{});

// Packed variable-length sequences (varlen.hip): the chunk table has
// varlen_slots(T, nseq, Q) int4 entries.
hipError_t launch_varlen_table(const int* cu, int nseq, int T, int Q, int4* tab, hipStream_t st);

// Element-wise stages next to the core (epilogue.hip).
hipError_t launch_gated_rmsnorm(ssd_dtype type, const void* y, const void* z, const float* w, void* out,
                                long ntok, int dim, int group, float eps, hipStream_t st);
hipError_t launch_causal_conv1d(ssd_dtype type, const void* x, const float* w, const float* bias,
                                const void* init, void* out, void* fin, int b, int T, int C, int K, int act,
                                hipStream_t st);
hipError_t launch_causal_conv1d_update(ssd_dtype type, void* state, const void* x, const float* w,
                                       const float* bias, void* out, int b, int C, int K, int act,
                                       hipStream_t st);

// ---------------------------------------------------------------------------
// Backward pass (bwd_chunk_mfma.hip, state_passing.hip, chunk_state_mfma.hip).
// The backward recomputes the forward with its own chunk length, the largest
// of 128, 64, 32 whose per-chunk tiles fit the 160 KB of LDS of a CU (x, dy,
// B, C rows of the chunk, the P x N state gradient and state in bf16, six
// per-token tables; the state's bf16 low part as well where it fits too), so one kernel serves each (headdim, dstate); 0: shape
// not supported. 128 at most: its work-group has 8 waves per 128 tokens, and
// 16-wave work-groups would leave 128 registers per lane, too few for the
// accumulators.
// ---------------------------------------------------------------------------
constexpr int kBwdLdsMax = 160 * 1024;
constexpr long bwd_lds_bytes(int P, int N, int Q) {
  return 4L * Q * (P + N) + 4L * P * N + 24L * Q;
}
constexpr int bwd_chunk_len(int P, int N) {
  return P * N > 128 * 128                        ? 0     // states beyond 64 KB in bf16: not supported
         : bwd_lds_bytes(P, N, 128) <= kBwdLdsMax ? 128
         : bwd_lds_bytes(P, N, 64) <= kBwdLdsMax  ? 64
         : bwd_lds_bytes(P, N, 32) <= kBwdLdsMax  ? 32
                                                  : 0;
}

// The forward recomputation for the backward: as launch_chunk_state_mfma (no
// chunk table), with the C B^T tiles in fp32 (CB [b, nc, G, ntile, 64, 16]
// f32) and also in the transposed orientation (CBt, lanes = s).
hipError_t launch_chunk_state_mfma_bwd(const FwdShape& s, const void* x, const void* B, const void* C,
                                       const void* dt, const float* A, float* Acs, float* dtq, float* S,
                                       uint16_t* CB, uint16_t* CBt, hipStream_t st);
// dS_c^T [b, nc, H, P, N] f32 = sum_l exp(Acs_l) dy_l C_l^T per chunk.
hipError_t launch_chunk_dstates_mfma(const FwdShape& s, const void* dy, const void* C, const void* dt,
                                     const float* A, float* dS, hipStream_t st);
// Reverse inter-chunk pass: G_c (bf16 [b, nc, H, P, N]), per-wave partials of
// <G_c, H_c> (ghp [b, H, nc, state_passing_bwd_partials]) and dinit.
int state_passing_bwd_partials(const FwdShape& s);
hipError_t launch_state_passing_bwd(const FwdShape& s, const float* dS, const float* Hst, const float* Acs,
                                    const float* dfinal, uint16_t* Gb, float* ghp, float* dinit, hipStream_t st);

struct BwdArgs {
  const void *x, *B, *C, *dy;
  const float *Acs, *dtq;
  const float* CB;       // fp32 C B^T tiles (lanes = l, as the forward's)
  const float* CBt;      // the same, transposed (lanes = s)
  const float* Hst;      // states entering each chunk, fp32 [b, nc, H, P, N]
  const uint16_t* Gb;    // gradients of the states leaving each chunk, bf16 [b, nc, H, P, N]
  const float* ghp;      // partials of <G_c, H_c>
  int nghp;              // partials per (b, h, c)
  const float *A, *D;
  void *dx, *ddt;        // bf16 [b, T, H, P], [b, T, H]
  void *dB, *dC;         // bf16 [b, T, G, N]
  int nslice;            // work-groups sharing one (batch, chunk, group): bwd_slices
  float *dBs, *dCs;      // nslice > 1: per-slice fp32 partials [nslice, b, T, G, N]
  float *tsds, *tsdst, *tsdd, *tsdl;   // per-token dots of each head, fp32 [b, H, nc, Q]
  float *dAp, *dDp;      // per-chunk fp32 partials [b, H, nc]
};
int bwd_slices(const FwdShape& s);
hipError_t launch_bwd_chunk(const FwdShape& s, const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_reduce(const FwdShape& s, const BwdArgs& a, float* dA, float* dD, hipStream_t st);

hipError_t launch_state_update(ssd_dtype type, float* state, const void* x, const void* dt,
                               const float* A, const void* B, const void* C, const float* D, void* y,
                               int batch, int H, int P, int N, int G, hipStream_t st);

}  // namespace ssd
