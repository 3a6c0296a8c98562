// ssd_api.hip -- the C ABI: host-side argument checks, workspace layout and the
// launch sequence. Every check runs before the first launch; on any error
// nothing is launched or written.
#include <cstdlib>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "ssd_backward.h"
#include "ssd_epilogue.h"
#include "ssd_internal.h"

using namespace ssd;

namespace {

bool is_chunk_ok(int q) { return q == 16 || q == 32 || q == 64 || q == 128 || q == 256; }

bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u); }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
  if (!a || !b || !abytes || !bbytes) return false;
  const Range ra = range_of(a, abytes), rb = range_of(b, bbytes);
  return ra.lo < rb.hi && rb.lo < ra.hi;
}

size_t esize(ssd_dtype t) { return t == SSD_BF16 ? 2 : 4; }

// SSD_DEBUG=1 in the environment: an entry point that launched work
// synchronises its stream before it returns, so a kernel that failed on the
// device is reported as SSD_ERR_HIP by the call that launched it instead of by
// the caller's next synchronisation (not for use under stream capture, where
// synchronising is not allowed). Read once per process.
bool debug_sync() {
  static const bool on = [] {
    const char* v = std::getenv("SSD_DEBUG");
    return v != nullptr && v[0] == '1';
  }();
  return on;
}
ssd_status launched(hipStream_t st) {
  if (!debug_sync()) return SSD_OK;
  const bool ok = hipStreamSynchronize(st) == hipSuccess && hipGetLastError() == hipSuccess;
  return ok ? SSD_OK : SSD_ERR_HIP;
}

ssd_status check_dims(int batch, int seqlen, int H, int P, int N, int G) {
  if (batch < 1 || seqlen < 1 || H < 1 || P < 1 || N < 1 || G < 1) return SSD_ERR_SHAPE;
  if (H % G) return SSD_ERR_SHAPE;
  if (P > SSD_MAX_HEADDIM || N > SSD_MAX_DSTATE) return SSD_ERR_SHAPE;
  // grid limits: chunks and batch rows go to grid.y / grid.z
  if (batch > 65535) return SSD_ERR_SHAPE;
  return SSD_OK;
}

bool dtype_ok(ssd_dtype t) { return t == SSD_F32 || t == SSD_BF16; }

FwdShape make_shape(int batch, int seqlen, int H, int P, int N, int G, int Q) {
  FwdShape s;
  s.b = batch; s.T = seqlen; s.H = H; s.P = P; s.N = N; s.G = G; s.Q = Q;
  s.nc = (seqlen + Q - 1) / Q;
  return s;
}

// The largest one-dimensional launch of the forward pass must stay below 2^32
// work-items (the grid limit). Work-items per launch, from the launchers:
//   chunk_cumsum      64 per (b, c, h) row
//   chunk_state_mfma  512 per (b, c, h), plus 64 per C B^T tile (lpc (lpc + 1) / 2
//                     tiles per (b, c, g)) rounded up to 512-thread work-groups
//   state_passing     256 per 16 x 64 tile of each (b, h) state, or one per
//                     state element when dstate % 4 != 0
//   chunk_scan_mfma   256 per (b, 256-token super-chunk, h)
// The generic kernels use three-dimensional grids and stay far below it.
bool grids_fit(const FwdShape& s, bool mfma) {
  const double lim = 4294967295.0;
  const double bch = double(s.b) * s.nc * s.H;
  const double bh = double(s.b) * s.H;
  const int lpc = s.Q / 32;
  double worst = 64.0 * bch;
  worst = std::max(worst, s.N % 4 == 0 ? 256.0 * bh * ((s.P + 15) / 16) * ((s.N + 63) / 64)
                                       : bh * s.P * s.N);
  if (mfma) {
    worst = std::max(worst, 64.0 * double(s.b) * s.nc * s.G * (lpc * (lpc + 1) / 2) + 4096.0 +
                                512.0 * bch);
    const int cps = 256 / s.Q;
    worst = std::max(worst, 256.0 * bh * ((s.nc + cps - 1) / cps));
  }
  return worst < lim;
}

// The forward's plan for the states entering each chunk (bf16 matrix-core
// path only; segments allowed)
ChainPlan fwd_plan(const FwdShape& s, bool mfma) {
  return mfma ? chunk_state_chain_plan(s, true) : ChainPlan{};
}

// Backward workspace (byte offsets, 256-byte aligned), chunk length
// bwd_chunk_len(P, N):
//   acs, dtq [b,H,nc,Q] f32; st [b,nc,H,P,N] f32 (chunk states, then the states
//   entering each chunk); ds [b,nc,H,P,N] f32 (absent where the reverse walk
//   forms the state gradients: it never stores them); gb [b,nc,H,P,N] bf16;
//   cb, cbt [b,nc,G,ntile,64,16] f32 (C B^T tiles, both orientations);
//   fin [b,H,N,P] f32; ghp [b,H,nc,nghp] f32;
//   dbs, dcs [nslice,b,T,G,N] f32 (only with nslice > 1); dap, ddp [b,H,nc] f32;
//   tok [4, b,H,nc,Q] f32 (per-token dots of each head)
struct BwdLayout {
  size_t acs, dtq, st, ds, gb, cb, cbt, fin, ghp, dbs, dcs, dap, ddp, tok, total;
};

BwdLayout bwd_layout(const FwdShape& s, int nghp, int nslice, bool rev_walk) {
  BwdLayout w;
  const size_t row = size_t(s.b) * s.H * s.nc * s.Q * sizeof(float);
  const size_t nst = size_t(s.b) * s.nc * s.H * s.N * s.P;
  const size_t lpc = size_t(s.Q) / 32, ntile = lpc * (lpc + 1) / 2;
  const size_t bhc = size_t(s.b) * s.H * s.nc;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes, 256); return at; };
  w.acs = take(row);
  w.dtq = take(row);
  w.st = take(nst * sizeof(float));
  w.ds = take(rev_walk ? 0 : nst * sizeof(float));
  w.gb = take(nst * sizeof(uint16_t));
  w.cb = take(size_t(s.b) * s.nc * s.G * ntile * 1024 * sizeof(float));
  w.cbt = take(size_t(s.b) * s.nc * s.G * ntile * 1024 * sizeof(float));
  w.fin = take(size_t(s.b) * s.H * s.N * s.P * sizeof(float));
  w.ghp = take(bhc * nghp * sizeof(float));
  const size_t part = nslice > 1 ? size_t(nslice) * s.b * s.T * s.G * s.N * sizeof(float) : 0;
  w.dbs = take(part);
  w.dcs = take(part);
  w.dap = take(bhc * sizeof(float));
  w.ddp = take(bhc * sizeof(float));
  w.tok = take(4 * row);
  w.total = o;
  return w;
}

// shapes the backward supports, and its launches within the grid limit
// (bwd_chunk_kernel: 4 Q work-items per (b, c, h); the reduction: one per
// 4 elements of dB)
bool bwd_supported(int batch, int seqlen, int H, int P, int N, int G, ssd_dtype dtype, FwdShape& s) {
  if (dtype != SSD_BF16) return false;
  const int Qb = bwd_chunk_len(P, N);
  if (Qb == 0) return false;
  s = make_shape(batch, seqlen, H, P, N, G, Qb);
  if (!use_mfma_path(s, dtype) || !grids_fit(s, true)) return false;
  const double bch = double(s.b) * s.nc * s.H;
  return 4.0 * Qb * bch < 4294967295.0 && double(batch) * seqlen * G * (N / 4) < 4294967295.0;
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch memory of the allocation-free forward (ssd_chunk_scan_fwd_noalloc):
// one array per GPU, in the code object, held until the process ends. In
// host code `scratch` names a host-side stand-in, not device memory: its
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is ever handed to a kernel.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];   // device address of `scratch` per device (set once)

// The current device's scratch address (looked up on the first call on the
// device); SSD_ERR_HIP when there is no usable device or the lookup fails.
ssd_status scratch_address(void** out) {
  *out = nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSD_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSD_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return SSD_OK;
}

}  // namespace

extern "C" {

const char* ssd_status_string(ssd_status status) {
  switch (status) {
    case SSD_OK: return "ok";
    case SSD_ERR_NULL: return "a required pointer is NULL";
    case SSD_ERR_SHAPE: return "unsupported or inconsistent dimensions";
    case SSD_ERR_DTYPE: return "unsupported dtype";
    case SSD_ERR_CHUNK: return "chunk_len must be one of 16, 32, 64, 128, 256";
    case SSD_ERR_WORKSPACE: return "workspace missing or too small";
    case SSD_ERR_HIP: return "HIP kernel launch failed";
    case SSD_ERR_ALIAS: return "an output overlaps an input";
    case SSD_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case SSD_ERR_VALUE: return "a scalar argument is out of range";
  }
  return "unknown status";
}

size_t ssd_chunk_scan_fwd_workspace(int batch, int seqlen, int nheads, int headdim, int dstate,
                                    int ngroups, int chunk_len, ssd_dtype dtype) {
  if (!dtype_ok(dtype) || !is_chunk_ok(chunk_len)) return 0;
  if (check_dims(batch, seqlen, nheads, headdim, dstate, ngroups) != SSD_OK) return 0;
  const FwdShape s = make_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_len);
  const bool mfma = use_mfma_path(s, dtype);
  if (s.nc > 65535 || !grids_fit(s, mfma)) return 0;
  return ws_layout(s, mfma, fwd_plan(s, mfma)).total;
}

int ssd_chunk_scan_fwd_fused_states(int batch, int seqlen, int nheads, int headdim, int dstate,
                                    int ngroups, int chunk_len, ssd_dtype dtype) {
  if (!dtype_ok(dtype) || !is_chunk_ok(chunk_len)) return 0;
  if (check_dims(batch, seqlen, nheads, headdim, dstate, ngroups) != SSD_OK) return 0;
  const FwdShape s = make_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_len);
  if (s.nc > 65535 || !use_mfma_path(s, dtype) || !grids_fit(s, true)) return 0;
  const ChainPlan pl = fwd_plan(s, true);
  return pl.ok ? pl.nseg : 0;
}

int ssd_chunk_scan_fwd_plan(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
                            int chunk_len, ssd_dtype dtype, int compute_units, int* seglen) {
  if (seglen) *seglen = 0;
  if (!dtype_ok(dtype) || !is_chunk_ok(chunk_len)) return 0;
  if (check_dims(batch, seqlen, nheads, headdim, dstate, ngroups) != SSD_OK) return 0;
  const FwdShape s = make_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_len);
  if (s.nc > 65535 || !use_mfma_path(s, dtype) || !grids_fit(s, true)) return 0;
  const ChainPlan pl = chunk_state_chain_plan_for(s, compute_units, true);
  if (!pl.ok) return 0;
  if (seglen) *seglen = pl.seglen;
  return pl.nseg;
}

ssd_status ssd_chunk_scan_fwd_timed(const void* x, const void* dt, const float* A, const void* B,
                                    const void* C, const float* D, const float* init_state,
                                    void* y, float* final_state, int batch, int seqlen,
                                    int nheads, int headdim, int dstate, int ngroups,
                                    int chunk_len, ssd_dtype dtype, void* workspace,
                                    size_t workspace_bytes, void* stream,
                                    void* const* stage_events) {
  if (!dtype_ok(dtype)) return SSD_ERR_DTYPE;
  ssd_status st = check_dims(batch, seqlen, nheads, headdim, dstate, ngroups);
  if (st != SSD_OK) return st;
  if (!is_chunk_ok(chunk_len)) return SSD_ERR_CHUNK;
  if (!x || !dt || !A || !B || !C || !y) return SSD_ERR_NULL;
  if (!workspace) return SSD_ERR_WORKSPACE;
  const void* ptrs[] = {x, dt, A, B, C, D, init_state, y, final_state, workspace};
  for (const void* p : ptrs)
    if (misaligned(p)) return SSD_ERR_ALIGN;

  const FwdShape s = make_shape(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_len);
  if (s.nc > 65535) return SSD_ERR_SHAPE;
  const bool mfma = use_mfma_path(s, dtype);
  if (!grids_fit(s, mfma)) return SSD_ERR_SHAPE;
  const ChainPlan pl = fwd_plan(s, mfma);
  const WsLayout w = ws_layout(s, mfma, pl);
  if (workspace_bytes < w.total) return SSD_ERR_WORKSPACE;

  const size_t e = esize(dtype);
  const size_t tok = size_t(batch) * seqlen;
  const size_t xb = tok * nheads * headdim * e, dtb = tok * nheads * e;
  const size_t bcb = tok * ngroups * dstate * e, hb = size_t(nheads) * sizeof(float);
  const size_t stb = size_t(batch) * nheads * dstate * headdim * sizeof(float);
  struct In {
    const void* p;
    size_t n;
  } ins[] = {{x, xb}, {dt, dtb}, {A, hb}, {B, bcb}, {C, bcb}, {D, hb}, {init_state, stb}};
  for (const In& in : ins) {
    if (overlaps(y, xb, in.p, in.n)) return SSD_ERR_ALIAS;
    if (overlaps(workspace, w.total, in.p, in.n)) return SSD_ERR_ALIAS;
    if (in.p != init_state && overlaps(final_state, stb, in.p, in.n)) return SSD_ERR_ALIAS;
  }
  if (overlaps(y, xb, final_state, stb) || overlaps(y, xb, workspace, w.total) ||
      overlaps(final_state, stb, workspace, w.total))
    return SSD_ERR_ALIAS;
  if (final_state && init_state && final_state != static_cast<const void*>(init_state) &&
      overlaps(final_state, stb, init_state, stb))
    return SSD_ERR_ALIAS;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* Acs = reinterpret_cast<float*>(ws + w.acs);
  float* dtq = reinterpret_cast<float*>(ws + w.dtq);
  float* S = reinterpret_cast<float*>(ws + w.st);
  uint16_t* Hb = mfma ? reinterpret_cast<uint16_t*>(ws + w.hb) : nullptr;
  uint16_t* CB = mfma ? reinterpret_cast<uint16_t*>(ws + w.cb) : nullptr;
  float* cdec = reinterpret_cast<float*>(ws + w.cdec);
  float* segdec = reinterpret_cast<float*>(ws + w.segdec);
  uint16_t* Cf = mfma ? reinterpret_cast<uint16_t*>(ws + w.cf) : nullptr;

  // stage i's events: stage_events[2 i] (start), stage_events[2 i + 1] (stop),
  // recorded by the kernel's own dispatch
  auto ev = [&](int i) {
    StageEv e;
    if (stage_events) {
      e.start = static_cast<hipEvent_t>(stage_events[2 * i]);
      e.stop = static_cast<hipEvent_t>(stage_events[2 * i + 1]);
    }
    return e;
  };
  // stage 0: cumulative sums, 1: chunk states, 2: state passing, 3: chunk
  // outputs. The matrix-core chunk_state launch also computes the cumulative
  // sums and the C B^T tiles, so stage 0 launches nothing on that path: its
  // two events are recorded back to back.
  if (mfma) {
    const StageEv e0 = ev(0);
    if (e0.start && hipEventRecord(e0.start, hs) != hipSuccess) return SSD_ERR_HIP;
    if (e0.stop && hipEventRecord(e0.stop, hs) != hipSuccess) return SSD_ERR_HIP;
  } else if (launch_chunk_cumsum(s, dtype, dt, A, Acs, dtq, hs, ev(0)) != hipSuccess) {
    return SSD_ERR_HIP;
  }
  if (pl.ok) {
    if (pl.nseg > 1) {
      // segmented walks (each segment's last local state into S), then the
      // recurrence over the segments: S[k] becomes the state entering segment
      // k, with segment k's summed decay exponent as its "chunk" decay (a
      // chunk length of 1 over segdec), from zero (segment 0 started from
      // init_state itself)
      if (launch_chunk_state_chain(s, pl, x, B, C, dt, A, Acs, dtq, Hb, init_state, S, CB, Cf, cdec, segdec, hs,
                                   ev(1)) != hipSuccess)
        return SSD_ERR_HIP;
      FwdShape ss = s;
      ss.nc = pl.nseg;
      ss.Q = 1;
      if (launch_state_passing(ss, S, nullptr, segdec, nullptr, final_state, hs, ev(2), true) != hipSuccess)
        return SSD_ERR_HIP;
      SegStates sg;
      sg.Hin = S;
      sg.cdec = cdec;
      sg.nseg = pl.nseg;
      sg.seglen = pl.seglen;
      if (launch_chunk_scan_mfma(s, x, CB, Cf, Acs, dtq, Hb, D, y, nullptr, hs, ev(3), sg) != hipSuccess)
        return SSD_ERR_HIP;
      return launched(hs);
    }
    // chunk states and state passing in one launch: stage 2 launches nothing
    if (launch_chunk_state_chain(s, pl, x, B, C, dt, A, Acs, dtq, Hb, init_state, final_state, CB, Cf, nullptr,
                                 nullptr, hs, ev(1)) != hipSuccess)
      return SSD_ERR_HIP;
    const StageEv e2 = ev(2);
    if (e2.start && hipEventRecord(e2.start, hs) != hipSuccess) return SSD_ERR_HIP;
    if (e2.stop && hipEventRecord(e2.stop, hs) != hipSuccess) return SSD_ERR_HIP;
  } else {
    const hipError_t se = mfma ? launch_chunk_state_mfma(s, x, B, C, dt, A, Acs, dtq, S, CB, Cf, nullptr, hs, ev(1))
                               : launch_chunk_state(s, dtype, x, B, Acs, dtq, S, hs, ev(1));
    if (se != hipSuccess) return SSD_ERR_HIP;
    if (launch_state_passing(s, S, Hb, Acs, init_state, final_state, hs, ev(2)) != hipSuccess)
      return SSD_ERR_HIP;
  }
  if (launch_chunk_scan(s, dtype, mfma, x, B, C, Acs, dtq, S, Hb, CB, Cf, D, y, hs, ev(3)) != hipSuccess)
    return SSD_ERR_HIP;
  return launched(hs);
}

ssd_status ssd_chunk_scan_fwd(const void* x, const void* dt, const float* A, const void* B,
                              const void* C, const float* D, const float* init_state, void* y,
                              float* final_state, int batch, int seqlen, int nheads, int headdim,
                              int dstate, int ngroups, int chunk_len, ssd_dtype dtype,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return ssd_chunk_scan_fwd_timed(x, dt, A, B, C, D, init_state, y, final_state, batch, seqlen,
                                  nheads, headdim, dstate, ngroups, chunk_len, dtype, workspace,
                                  workspace_bytes, stream, nullptr);
}

ssd_status ssd_chunk_scan_fwd_noalloc(const void* x, const void* dt, const float* A, const void* B,
                                      const void* C, const float* D, const float* init_state, void* y,
                                      float* final_state, int batch, int seqlen, int nheads, int headdim,
                                      int dstate, int ngroups, int chunk_len, ssd_dtype dtype, void* stream) {
  void* ws = nullptr;
  const ssd_status st = scratch_address(&ws);
  if (st != SSD_OK) return st;
  // the same checks and launches as ssd_chunk_scan_fwd, over this device's
  // scratch: sizes whose workspace exceeds it return SSD_ERR_WORKSPACE before
  // any launch; every byte of it that a call reads, the call writes first
  return ssd_chunk_scan_fwd_timed(x, dt, A, B, C, D, init_state, y, final_state, batch, seqlen, nheads, headdim,
                                  dstate, ngroups, chunk_len, dtype, ws, SSD_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

ssd_status ssd_state_update(float* state, const void* x, const void* dt, const float* A,
                            const void* B, const void* C, const float* D, void* y, int batch,
                            int nheads, int headdim, int dstate, int ngroups, ssd_dtype dtype,
                            void* stream) {
  if (!dtype_ok(dtype)) return SSD_ERR_DTYPE;
  ssd_status st = check_dims(batch, 1, nheads, headdim, dstate, ngroups);
  if (st != SSD_OK) return st;
  if (!state || !x || !dt || !A || !B || !C || !y) return SSD_ERR_NULL;
  const void* ptrs[] = {state, x, dt, A, B, C, D, y};
  for (const void* p : ptrs)
    if (misaligned(p)) return SSD_ERR_ALIGN;
  const size_t e = esize(dtype);
  const size_t xb = size_t(batch) * nheads * headdim * e, dtb = size_t(batch) * nheads * e;
  const size_t bcb = size_t(batch) * ngroups * dstate * e, hb = size_t(nheads) * sizeof(float);
  const size_t stb = size_t(batch) * nheads * dstate * headdim * sizeof(float);
  struct In {
    const void* p;
    size_t n;
  } ins[] = {{x, xb}, {dt, dtb}, {A, hb}, {B, bcb}, {C, bcb}, {D, hb}};
  for (const In& in : ins) {
    if (overlaps(y, xb, in.p, in.n)) return SSD_ERR_ALIAS;
    if (overlaps(state, stb, in.p, in.n)) return SSD_ERR_ALIAS;
  }
  if (overlaps(y, xb, state, stb)) return SSD_ERR_ALIAS;
  if (launch_state_update(dtype, state, x, dt, A, B, C, D, y, batch, nheads, headdim, dstate,
                          ngroups, static_cast<hipStream_t>(stream)) != hipSuccess)
    return SSD_ERR_HIP;
  return launched(static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------
// packed variable-length sequences
// ---------------------------------------------------------------------------
namespace {
// one batch row of `total` tokens cut into table slots
FwdShape varlen_shape(int total, int nseq, int H, int P, int N, int G, int Q) {
  FwdShape s = make_shape(1, total, H, P, N, G, Q);
  s.nc = varlen_slots(total, nseq, Q);
  return s;
}
// Workspace of a packed call: the forward's layout for one row of chunk
// slots (with the fused walk's segments where the plan has them: segment
// states, cdec, segdec), then with the walk F [nseg, H, P * N] f32, fdec
// [H, nseg] f32 and fseq [nseg] int32 (the segments' first sequences that
// end inside them), then the chunk table.
struct VarlenWs {
  WsLayout w;
  size_t F, fdec, fseq, tab, total;
};
VarlenWs varlen_ws(const FwdShape& s, const ChainPlan& pl) {
  VarlenWs v;
  v.w = ws_layout(s, true, pl);
  const size_t nsg = pl.ok ? size_t(pl.nseg) : 0;
  v.F = align_up(v.w.total, 256);
  v.fdec = align_up(v.F + nsg * s.H * s.P * s.N * sizeof(float), 256);
  v.fseq = align_up(v.fdec + nsg * s.H * sizeof(float), 256);
  v.tab = align_up(v.fseq + nsg * sizeof(int), 256);
  v.total = v.tab + size_t(s.nc) * sizeof(int4);
  return v;
}
// the per-sequence state passing launches 256 threads per (sequence, head,
// 16 x 64 state tile)
bool varlen_grids_fit(const FwdShape& s, int nseq) {
  return grids_fit(s, true) &&
         256.0 * nseq * s.H * ((s.P + 15) / 16) * ((s.N + 63) / 64) < 4294967295.0;
}
}  // namespace

size_t ssd_chunk_scan_fwd_varlen_workspace(int total_tokens, int nseq, int nheads, int headdim, int dstate,
                                           int ngroups, int chunk_len, ssd_dtype dtype) {
  if (!dtype_ok(dtype) || !is_chunk_ok(chunk_len) || nseq < 1 || nseq > 65535) return 0;
  if (check_dims(1, total_tokens, nheads, headdim, dstate, ngroups) != SSD_OK) return 0;
  const FwdShape s = varlen_shape(total_tokens, nseq, nheads, headdim, dstate, ngroups, chunk_len);
  if (!use_mfma_path(s, dtype) || !varlen_grids_fit(s, nseq)) return 0;
  return varlen_ws(s, varlen_chain_plan_for(s, nseq, device_units())).total;
}

int ssd_chunk_scan_fwd_varlen_plan(int total_tokens, int nseq, int nheads, int headdim, int dstate, int ngroups,
                                   int chunk_len, ssd_dtype dtype, int compute_units, int* seglen) {
  if (seglen) *seglen = 0;
  if (!dtype_ok(dtype) || !is_chunk_ok(chunk_len) || nseq < 1 || nseq > 65535) return 0;
  if (check_dims(1, total_tokens, nheads, headdim, dstate, ngroups) != SSD_OK) return 0;
  const FwdShape s = varlen_shape(total_tokens, nseq, nheads, headdim, dstate, ngroups, chunk_len);
  if (!use_mfma_path(s, dtype) || !varlen_grids_fit(s, nseq)) return 0;
  const ChainPlan pl = varlen_chain_plan_for(s, nseq, compute_units);
  if (!pl.ok) return 0;
  if (seglen) *seglen = pl.seglen;
  return pl.nseg;
}

ssd_status ssd_chunk_scan_fwd_varlen(const void* x, const void* dt, const float* A, const void* B,
                                     const void* C, const float* D, const int* cu_seqlens,
                                     const float* init_states, void* y, float* final_states,
                                     int total_tokens, int nseq, int nheads, int headdim, int dstate,
                                     int ngroups, int chunk_len, ssd_dtype dtype, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return SSD_ERR_DTYPE;
  ssd_status st = check_dims(1, total_tokens, nheads, headdim, dstate, ngroups);
  if (st != SSD_OK) return st;
  if (nseq < 1 || nseq > 65535) return SSD_ERR_SHAPE;
  if (!is_chunk_ok(chunk_len)) return SSD_ERR_CHUNK;
  if (!x || !dt || !A || !B || !C || !y || !cu_seqlens) return SSD_ERR_NULL;
  if (!workspace) return SSD_ERR_WORKSPACE;
  const void* ptrs[] = {x, dt, A, B, C, D, init_states, y, final_states, workspace};
  for (const void* p : ptrs)
    if (misaligned(p)) return SSD_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) return SSD_ERR_ALIGN;
  const FwdShape s = varlen_shape(total_tokens, nseq, nheads, headdim, dstate, ngroups, chunk_len);
  if (!use_mfma_path(s, dtype) || !varlen_grids_fit(s, nseq)) return SSD_ERR_SHAPE;
  const ChainPlan pl = varlen_chain_plan_for(s, nseq, device_units());
  const VarlenWs v = varlen_ws(s, pl);
  const WsLayout& w = v.w;
  if (workspace_bytes < v.total) return SSD_ERR_WORKSPACE;

  const size_t e = esize(dtype);
  const size_t tok = size_t(total_tokens);
  const size_t xb = tok * nheads * headdim * e, dtb = tok * nheads * e;
  const size_t bcb = tok * ngroups * dstate * e, hb = size_t(nheads) * sizeof(float);
  const size_t stb = size_t(nseq) * nheads * dstate * headdim * sizeof(float);
  const size_t cub = size_t(nseq + 1) * sizeof(int);
  const size_t wsb = v.total;
  struct In {
    const void* p;
    size_t n;
  } ins[] = {{x, xb}, {dt, dtb}, {A, hb}, {B, bcb}, {C, bcb}, {D, hb}, {init_states, stb}, {cu_seqlens, cub}};
  for (const In& in : ins) {
    if (overlaps(y, xb, in.p, in.n) || overlaps(workspace, wsb, in.p, in.n)) return SSD_ERR_ALIAS;
    if (in.p != init_states && overlaps(final_states, stb, in.p, in.n)) return SSD_ERR_ALIAS;
  }
  if (overlaps(y, xb, final_states, stb) || overlaps(y, xb, workspace, wsb) ||
      overlaps(final_states, stb, workspace, wsb))
    return SSD_ERR_ALIAS;
  if (final_states && init_states && final_states != init_states && overlaps(final_states, stb, init_states, stb))
    return SSD_ERR_ALIAS;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* Acs = reinterpret_cast<float*>(ws + w.acs);
  float* dtq = reinterpret_cast<float*>(ws + w.dtq);
  float* S = reinterpret_cast<float*>(ws + w.st);
  uint16_t* Hb = reinterpret_cast<uint16_t*>(ws + w.hb);
  uint16_t* CB = reinterpret_cast<uint16_t*>(ws + w.cb);
  uint16_t* Cf = reinterpret_cast<uint16_t*>(ws + w.cf);
  int4* tab = reinterpret_cast<int4*>(ws + v.tab);
  if (launch_varlen_table(cu_seqlens, nseq, total_tokens, chunk_len, tab, hs) != hipSuccess) return SSD_ERR_HIP;
  if (pl.ok) {
    // the fused walk over equal segments of the slot row, restarting at each
    // sequence's first chunk; the recurrence over the segments (states
    // entering them, the final states of sequences that cross a segment
    // boundary, empty sequences); chunk_scan with the segment correction.
    // A sequence's initial state is read by the walk that holds its first
    // chunk before the final state is written (by the same walk, or by the
    // recurrence after it; an empty sequence's by the recurrence, element by
    // element), so final_states may be init_states.
    float* cdec = reinterpret_cast<float*>(ws + w.cdec);
    float* segdec = reinterpret_cast<float*>(ws + w.segdec);
    VarWalk vw;
    vw.tab = tab;
    vw.nseq = nseq;
    vw.fin = final_states;
    vw.F = reinterpret_cast<float*>(ws + v.F);
    vw.fdec = reinterpret_cast<float*>(ws + v.fdec);
    vw.fseq = reinterpret_cast<int*>(ws + v.fseq);
    if (launch_chunk_state_chain_varlen(s, pl, x, B, C, dt, A, Acs, dtq, Hb, init_states, S, CB, Cf, cdec, segdec,
                                        vw, hs) != hipSuccess)
      return SSD_ERR_HIP;
    FwdShape ss = s;
    ss.nc = pl.nseg;
    if (launch_varlen_segment_recurrence(ss, S, vw.F, segdec, vw.fdec, vw.fseq, cu_seqlens, nseq, init_states,
                                         final_states, hs) != hipSuccess)
      return SSD_ERR_HIP;
    SegStates sg;
    sg.Hin = S;
    sg.cdec = cdec;
    sg.nseg = pl.nseg;
    sg.seglen = pl.seglen;
    sg.var = true;
    if (launch_chunk_scan_mfma(s, x, CB, Cf, Acs, dtq, Hb, D, y, tab, hs, StageEv{}, sg) != hipSuccess)
      return SSD_ERR_HIP;
    return launched(hs);
  }
  // per chunk: chunk states, the recurrence per sequence, chunk_scan.
  // state_passing reads each sequence's initial state (whole tile, into
  // LDS) before it writes that sequence's final state, so final_states may
  // be init_states.
  if (launch_chunk_state_mfma(s, x, B, C, dt, A, Acs, dtq, S, CB, Cf, tab, hs) != hipSuccess) return SSD_ERR_HIP;
  if (launch_state_passing_varlen(s, S, Hb, Acs, cu_seqlens, nseq, init_states, final_states, hs) != hipSuccess)
    return SSD_ERR_HIP;
  if (launch_chunk_scan_mfma(s, x, CB, Cf, Acs, dtq, Hb, D, y, tab, hs) != hipSuccess) return SSD_ERR_HIP;
  return launched(hs);
}

ssd_status ssd_gated_rmsnorm(const void* y, const void* z, const float* weight, void* out, long ntokens,
                             int dim, int group, float eps, ssd_dtype dtype, void* stream) {
  if (!dtype_ok(dtype)) return SSD_ERR_DTYPE;
  if (ntokens < 1 || dim < 1 || group < 1 || dim % group) return SSD_ERR_SHAPE;
  const double rows = double(ntokens) * (dim / group);
  if (rows > double(1L << 26)) return SSD_ERR_SHAPE;     // one wave per row, 64 lanes each
  if (!(eps >= 0.f) || !std::isfinite(eps)) return SSD_ERR_VALUE;
  if (!y || !z || !weight || !out) return SSD_ERR_NULL;
  const void* ptrs[] = {y, z, weight, out};
  for (const void* p : ptrs)
    if (misaligned(p)) return SSD_ERR_ALIGN;
  const size_t nb = size_t(ntokens) * dim * esize(dtype), wb = size_t(dim) * sizeof(float);
  if (out != y && overlaps(out, nb, y, nb)) return SSD_ERR_ALIAS;
  if (overlaps(out, nb, z, nb) || overlaps(out, nb, weight, wb)) return SSD_ERR_ALIAS;
  if (launch_gated_rmsnorm(dtype, y, z, weight, out, ntokens, dim, group, eps,
                           static_cast<hipStream_t>(stream)) != hipSuccess)
    return SSD_ERR_HIP;
  return launched(static_cast<hipStream_t>(stream));
}

ssd_status ssd_causal_conv1d_fwd(const void* x, const float* weight, const float* bias,
                                 const void* init_state, void* out, void* final_state, int batch,
                                 int seqlen, int channels, int kernel_width, int activation,
                                 ssd_dtype dtype, void* stream) {
  if (!dtype_ok(dtype)) return SSD_ERR_DTYPE;
  if (batch < 1 || seqlen < 1 || channels < 1 || kernel_width < 1 || kernel_width > SSD_CONV_MAX_WIDTH)
    return SSD_ERR_SHAPE;
  if (double(batch) * ((seqlen + 15) / 16) * channels > double(0x7fffffff)) return SSD_ERR_SHAPE;
  if (activation != 0 && activation != 1) return SSD_ERR_VALUE;
  if (!x || !weight || !out) return SSD_ERR_NULL;
  const void* ptrs[] = {x, weight, bias, init_state, out, final_state};
  for (const void* p : ptrs)
    if (misaligned(p)) return SSD_ERR_ALIGN;
  const size_t e = esize(dtype);
  const size_t xb = size_t(batch) * seqlen * channels * e;
  const size_t sb = size_t(batch) * (kernel_width - 1) * channels * e;
  const size_t wb = size_t(channels) * kernel_width * sizeof(float), bb = size_t(channels) * sizeof(float);
  struct In {
    const void* p;
    size_t n;
  } ins[] = {{x, xb}, {weight, wb}, {bias, bb}, {init_state, sb}, {final_state, sb}};
  for (const In& in : ins)
    if (overlaps(out, xb, in.p, in.n)) return SSD_ERR_ALIAS;
  if (final_state && sb) {
    if (overlaps(final_state, sb, x, xb) || overlaps(final_state, sb, weight, wb) ||
        overlaps(final_state, sb, bias, bb))
      return SSD_ERR_ALIAS;
    if (final_state != init_state && overlaps(final_state, sb, init_state, sb)) return SSD_ERR_ALIAS;
  }
  if (launch_causal_conv1d(dtype, x, weight, bias, init_state, out, sb ? final_state : nullptr, batch,
                           seqlen, channels, kernel_width, activation,
                           static_cast<hipStream_t>(stream)) != hipSuccess)
    return SSD_ERR_HIP;
  return launched(static_cast<hipStream_t>(stream));
}

ssd_status ssd_causal_conv1d_update(void* state, const void* x, const float* weight, const float* bias,
                                    void* out, int batch, int channels, int kernel_width, int activation,
                                    ssd_dtype dtype, void* stream) {
  if (!dtype_ok(dtype)) return SSD_ERR_DTYPE;
  if (batch < 1 || channels < 1 || kernel_width < 1 || kernel_width > SSD_CONV_MAX_WIDTH)
    return SSD_ERR_SHAPE;
  if (double(batch) * channels > double(0x7fffffff)) return SSD_ERR_SHAPE;
  if (activation != 0 && activation != 1) return SSD_ERR_VALUE;
  if (!x || !weight || !out || (!state && kernel_width > 1)) return SSD_ERR_NULL;
  const void* ptrs[] = {state, x, weight, bias, out};
  for (const void* p : ptrs)
    if (misaligned(p)) return SSD_ERR_ALIGN;
  const size_t e = esize(dtype);
  const size_t xb = size_t(batch) * channels * e;
  const size_t sb = size_t(batch) * (kernel_width - 1) * channels * e;
  const size_t wb = size_t(channels) * kernel_width * sizeof(float), bb = size_t(channels) * sizeof(float);
  struct In {
    const void* p;
    size_t n;
  } ins[] = {{x, xb}, {weight, wb}, {bias, bb}};
  for (const In& in : ins)
    if (overlaps(out, xb, in.p, in.n) || overlaps(state, sb, in.p, in.n)) return SSD_ERR_ALIAS;
  if (overlaps(out, xb, state, sb)) return SSD_ERR_ALIAS;
  if (launch_causal_conv1d_update(dtype, state, x, weight, bias, out, batch, channels, kernel_width,
                                  activation, static_cast<hipStream_t>(stream)) != hipSuccess)
    return SSD_ERR_HIP;
  return launched(static_cast<hipStream_t>(stream));
}

size_t ssd_chunk_scan_bwd_workspace(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
                                    ssd_dtype dtype) {
  if (!dtype_ok(dtype) || check_dims(batch, seqlen, nheads, headdim, dstate, ngroups) != SSD_OK) return 0;
  FwdShape s;
  if (!bwd_supported(batch, seqlen, nheads, headdim, dstate, ngroups, dtype, s)) return 0;
  return bwd_layout(s, state_passing_bwd_partials(s), bwd_slices(s), chunk_grad_chain_ok(s)).total;
}

int ssd_chunk_scan_bwd_fused_walks(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
                                   ssd_dtype dtype) {
  if (!dtype_ok(dtype) || check_dims(batch, seqlen, nheads, headdim, dstate, ngroups) != SSD_OK) return 0;
  FwdShape s;
  if (!bwd_supported(batch, seqlen, nheads, headdim, dstate, ngroups, dtype, s)) return 0;
  return (chunk_state_chain_ok(s) ? 1 : 0) | (chunk_grad_chain_ok(s) ? 2 : 0);
}

ssd_status ssd_chunk_scan_bwd(const void* x, const void* dt, const float* A, const void* B, const void* C,
                              const float* D, const float* init_state, const void* dy, const float* dfinal,
                              void* dx, void* ddt, float* dA, void* dB, void* dC, float* dD, float* dinit,
                              int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
                              ssd_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return SSD_ERR_DTYPE;
  ssd_status st = check_dims(batch, seqlen, nheads, headdim, dstate, ngroups);
  if (st != SSD_OK) return st;
  FwdShape s;
  if (!bwd_supported(batch, seqlen, nheads, headdim, dstate, ngroups, dtype, s)) return SSD_ERR_SHAPE;
  if (!x || !dt || !A || !B || !C || !dy || !dx || !ddt || !dA || !dB || !dC) return SSD_ERR_NULL;
  if (!workspace) return SSD_ERR_WORKSPACE;
  const void* ptrs[] = {x, dt, A, B, C, D, init_state, dy, dfinal, dx, ddt, dA, dB, dC, dD, dinit, workspace};
  for (const void* p : ptrs)
    if (misaligned(p)) return SSD_ERR_ALIGN;
  const int nghp = state_passing_bwd_partials(s);
  const int nslice = bwd_slices(s);
  const bool rev_walk = chunk_grad_chain_ok(s);
  const BwdLayout w = bwd_layout(s, nghp, nslice, rev_walk);
  if (workspace_bytes < w.total) return SSD_ERR_WORKSPACE;

  const size_t e = esize(dtype);
  const size_t tok = size_t(batch) * seqlen;
  const size_t xb = tok * nheads * headdim * e, dtb = tok * nheads * e, bcb = tok * ngroups * dstate * e;
  const size_t hb = size_t(nheads) * sizeof(float);
  const size_t stb = size_t(batch) * nheads * dstate * headdim * sizeof(float);
  struct Buf {
    const void* p;
    size_t n;
  };
  const Buf ins[] = {{x, xb}, {dt, dtb}, {A, hb}, {B, bcb}, {C, bcb}, {D, hb}, {init_state, stb}, {dy, xb},
                     {dfinal, stb}, {workspace, w.total}};
  const Buf outs[] = {{dx, xb}, {ddt, dtb}, {dA, hb}, {dB, bcb}, {dC, bcb}, {dD, hb}, {dinit, stb}};
  for (const Buf& o : outs) {
    for (const Buf& in : ins)
      if (overlaps(o.p, o.n, in.p, in.n)) return SSD_ERR_ALIAS;
    for (const Buf& o2 : outs)
      if (&o2 != &o && overlaps(o.p, o.n, o2.p, o2.n)) return SSD_ERR_ALIAS;
  }

  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* Acs = reinterpret_cast<float*>(ws + w.acs);
  float* dtq = reinterpret_cast<float*>(ws + w.dtq);
  float* Sst = reinterpret_cast<float*>(ws + w.st);
  float* dS = reinterpret_cast<float*>(ws + w.ds);
  uint16_t* Gb = reinterpret_cast<uint16_t*>(ws + w.gb);
  uint16_t* CBf = reinterpret_cast<uint16_t*>(ws + w.cb);
  uint16_t* CBt = reinterpret_cast<uint16_t*>(ws + w.cbt);
  float* fin = reinterpret_cast<float*>(ws + w.fin);
  float* ghp = reinterpret_cast<float*>(ws + w.ghp);
  float* dBs = reinterpret_cast<float*>(ws + w.dbs);
  float* dCs = reinterpret_cast<float*>(ws + w.dcs);
  float* dAp = reinterpret_cast<float*>(ws + w.dap);
  float* dDp = reinterpret_cast<float*>(ws + w.ddp);

  // recomputation: in-chunk decays, chunk states, then the states entering
  // each chunk (fp32, over the chunk states) and the final state -- in one
  // launch where the fused walk applies
  if (chunk_state_chain_ok(s)) {
    if (launch_chunk_state_chain_bwd(s, x, B, C, dt, A, Acs, dtq, Sst, init_state, fin, CBf, CBt, hs) !=
        hipSuccess)
      return SSD_ERR_HIP;
  } else {
    if (launch_chunk_state_mfma_bwd(s, x, B, C, dt, A, Acs, dtq, Sst, CBf, CBt, hs) != hipSuccess)
      return SSD_ERR_HIP;
    if (launch_state_passing(s, Sst, nullptr, Acs, init_state, fin, hs) != hipSuccess) return SSD_ERR_HIP;
  }
  // what each chunk's outputs give the state entering it, then the reverse
  // pass -- in one reverse walk where the fused walk applies
  if (rev_walk) {
    if (launch_chunk_grad_chain_bwd(s, dy, C, dt, A, dfinal, Gb, dinit, Sst, ghp, hs) != hipSuccess)
      return SSD_ERR_HIP;
  } else {
    if (launch_chunk_dstates_mfma(s, dy, C, dt, A, dS, hs) != hipSuccess) return SSD_ERR_HIP;
    if (launch_state_passing_bwd(s, dS, Sst, Acs, dfinal, Gb, ghp, dinit, hs) != hipSuccess)
      return SSD_ERR_HIP;
  }
  BwdArgs a;
  a.x = x; a.B = B; a.C = C; a.dy = dy; a.Acs = Acs; a.dtq = dtq; a.CB = reinterpret_cast<const float*>(CBf); a.CBt = reinterpret_cast<const float*>(CBt); a.Hst = Sst; a.Gb = Gb;
  a.ghp = ghp; a.nghp = rev_walk ? s.P / 16 : nghp;   // the reverse walk's partials per (b, h, c)
  a.A = A; a.D = D; a.dx = dx; a.ddt = ddt; a.dB = dB; a.dC = dC;
  a.nslice = nslice; a.dBs = dBs; a.dCs = dCs; a.dAp = dAp; a.dDp = dDp;
  float* tokd = reinterpret_cast<float*>(ws + w.tok);
  const size_t rowf = size_t(s.b) * s.H * s.nc * s.Q;
  a.tsds = tokd; a.tsdst = tokd + rowf; a.tsdd = tokd + 2 * rowf; a.tsdl = tokd + 3 * rowf;
  if (launch_bwd_chunk(s, a, hs) != hipSuccess) return SSD_ERR_HIP;
  if (launch_bwd_reduce(s, a, dA, dD, hs) != hipSuccess) return SSD_ERR_HIP;
  return launched(hs);
}

}  // extern "C"
