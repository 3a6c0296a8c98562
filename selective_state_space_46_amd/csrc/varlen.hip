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

constexpr int kTabThreads = 1024;

// one work-group: clear every slot, then each thread writes the entries of
// sequences tid, tid + 1024, ... (varlen_fill: slots < nslots for any clamped
// span)
__global__ __launch_bounds__(kTabThreads) void varlen_table_kernel(const int* __restrict__ cu, int nseq,
                                                                   int T, int Q, int nslots,
                                                                   int4* __restrict__ tab) {
  const int tid = threadIdx.x;
  for (int c = tid; c < nslots; c += kTabThreads) tab[c] = int4{0, 0, 0, 0};
  __syncthreads();   // the clears are ordered before the entries below
  for (int i = tid; i < nseq; i += kTabThreads) {
    int s0, len;
    varlen_span(cu, i, T, s0, len);
    varlen_fill(i, s0, len, Q, tab, nslots);
  }
}

}  // namespace

hipError_t launch_varlen_table(const int* cu, int nseq, int T, int Q, int4* tab, hipStream_t st) {
  hipLaunchKernelGGL(varlen_table_kernel, dim3(1), dim3(kTabThreads), 0, st, cu, nseq, T, Q,
                     varlen_slots(T, nseq, Q), tab);
  return hipGetLastError();
}

}  // namespace ssd
