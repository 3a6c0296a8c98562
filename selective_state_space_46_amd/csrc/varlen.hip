// varlen.hip -- packed variable-length sequences: the chunk table.
//
// Sequences packed along one token axis (sequence i is tokens cu[i] ..
// cu[i+1]-1) each start from their own state (youngju.dev "Mamba / selective
// SSM" page, section "状態初期化とシーケンス境界": the state is set explicitly
// at the start of every sequence so that the sequences of a batch never mix).
// The forward kernels run on chunks that each lie inside one sequence: a
// sequence of length L has ceil(L / Q) chunks, its last one holding L mod Q
// valid tokens (or Q). Chunk k of sequence i takes slot floor(cu[i] / Q) +
// i + k (ssd_internal.h), so a sequence's slots follow from its own offset
// alone; the table lists, for the kernels that walk slots, every slot's
// first token row, valid tokens, sequence and first/last flags. Slots that
// no chunk takes stay {0, 0, 0, 0}.
//
// cu_seqlens lives on the device and is not seen by the host, so the spans
// are clamped (varlen_span): malformed offsets give unspecified but
// in-bounds results.
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kTabThreads = 256;
constexpr int kTabLds = 4096;   // sequences whose first slots are staged in LDS

// one thread per slot, each writing its whole entry (varlen_slot_entry), so
// no slot needs clearing first and no thread walks a sequence's chunks in
// turn; up to kTabLds sequences, each work-group stages the sequences' first
// slots in LDS for the bisection, else it reads the offsets from memory
__global__ __launch_bounds__(kTabThreads) void varlen_table_kernel(const int* __restrict__ cu, int nseq,
                                                                   int T, int Q, int nslots,
                                                                   int4* __restrict__ tab) {
  __shared__ int sfirst[kTabLds];
  const int tid = threadIdx.x;
  const int c = int(blockIdx.x) * kTabThreads + tid;
  int4 e;
  if (nseq <= kTabLds) {
    for (int i = tid; i < nseq; i += kTabThreads) sfirst[i] = varlen_first_slot(clamp_int(cu[i], 0, T), i, Q);
    __syncthreads();
    if (c >= nslots) return;
    e = varlen_slot_entry(cu, nseq, T, Q, c, [&](int i) { return sfirst[i]; });
  } else {
    if (c >= nslots) return;
    e = varlen_slot_entry(cu, nseq, T, Q, c, [&](int i) { return varlen_first_slot(clamp_int(cu[i], 0, T), i, Q); });
  }
  tab[c] = e;
}

}  // namespace

hipError_t launch_varlen_table(const int* cu, int nseq, int T, int Q, int4* tab, hipStream_t st) {
  const int nslots = varlen_slots(T, nseq, Q);
  hipLaunchKernelGGL(varlen_table_kernel, dim3(unsigned((nslots + kTabThreads - 1) / kTabThreads)),
                     dim3(kTabThreads), 0, st, cu, nseq, T, Q, nslots, tab);
  return hipGetLastError();
}

}  // namespace ssd
