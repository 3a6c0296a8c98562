// varlen.hip -- packed variable-length sequences: the chunk table.
//
// Sequences packed along one token axis (sequence i is tokens cu[i] ..
// cu[i+1]-1) each start from their own state (youngju.dev "Mamba / selective
// SSM" page, section "状態初期化とシーケンス境界": the state is set explicitly
// at the start of every sequence so that the sequences of a batch never mix).
// The forward kernels run on chunks that each lie inside one sequence: a
// sequence of length L takes ceil(L / Q) chunk slots, its last chunk holding
// L mod Q valid tokens (or Q). The table gives every slot its first token
// row, valid tokens, sequence and first/last flags (see ChunkRows in
// ssd_internal.h); slots past the last chunk stay {0, 0, 0, 0}. There are at
// most ceil(T / Q) + nseq chunks.
//
// cu_seqlens lives on the device and is not seen by the host, so the table
// kernel clamps it: sequence i covers [clamp(cu[i]), max(that, clamp(cu[i+1])))
// with clamp to [0, T], and chunks beyond the slot count are dropped.
// Well-formed offsets (0 = cu[0] <= ... <= cu[nseq] = T) are used as given;
// malformed ones give unspecified (but in-bounds) results.
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kTabThreads = 1024;

__device__ __forceinline__ void seq_span(const int* cu, int i, int T, int& s0, int& len) {
  s0 = min(max(cu[i], 0), T);
  const int s1 = max(s0, min(max(cu[i + 1], 0), T));
  len = s1 - s0;
}

// one work-group: clear the slots, then each thread takes sequences
// base + tid, a work-group exclusive scan of their chunk counts gives their
// first slots
__global__ __launch_bounds__(kTabThreads) void varlen_table_kernel(const int* __restrict__ cu, int nseq,
                                                                   int T, int Q, int nslots,
                                                                   int4* __restrict__ tab) {
  __shared__ int scan[kTabThreads];
  const int tid = threadIdx.x;
  for (int c = tid; c < nslots; c += kTabThreads) tab[c] = int4{0, 0, 0, 0};
  __syncthreads();   // the clears are ordered before the entries below
  int carry = 0;
  for (int base = 0; base < nseq; base += kTabThreads) {
    const int i = base + tid;
    int s0 = 0, len = 0;
    if (i < nseq) seq_span(cu, i, T, s0, len);
    const int nch = (len + Q - 1) / Q;
    scan[tid] = nch;
    __syncthreads();
    for (int off = 1; off < kTabThreads; off <<= 1) {   // inclusive scan (Hillis-Steele)
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int first = carry + scan[tid] - nch;
    for (int k = 0; k < nch; ++k) {
      const int c = first + k;
      if (c >= nslots) break;
      const int flags = (k == 0 ? 1 : 0) | (k == nch - 1 ? 2 : 0);
      tab[c] = int4{s0 + k * Q, min(Q, len - k * Q), i, flags};
    }
    carry += scan[kTabThreads - 1];
    __syncthreads();   // scan[] is reused by the next group of sequences
  }
}

// sequences with no tokens: final state = initial state (or zero)
__global__ __launch_bounds__(256) void varlen_empty_finals(const int* __restrict__ cu, int nseq, int T,
                                                           const float* __restrict__ init,
                                                           float* __restrict__ fin, long per_seq) {
  const int i = blockIdx.y;
  int s0 = 0, len = 0;
  seq_span(cu, i, T, s0, len);
  if (len > 0) return;
  for (long e = long(blockIdx.x) * 256 + threadIdx.x; e < per_seq; e += long(gridDim.x) * 256)
    fin[size_t(i) * per_seq + e] = init ? init[size_t(i) * per_seq + e] : 0.f;
}

}  // namespace

int varlen_slots(int T, int nseq, int Q) { return (T + Q - 1) / Q + nseq; }

hipError_t launch_varlen_table(const int* cu, int nseq, int T, int Q, int4* tab, hipStream_t st) {
  hipLaunchKernelGGL(varlen_table_kernel, dim3(1), dim3(kTabThreads), 0, st, cu, nseq, T, Q,
                     varlen_slots(T, nseq, Q), tab);
  return hipGetLastError();
}

hipError_t launch_varlen_empty_finals(const int* cu, int nseq, int T, const float* init, float* fin,
                                      long per_seq, hipStream_t st) {
  const long want = (per_seq + 255) / 256;
  const unsigned gx = unsigned(want < 64 ? want : 64);
  hipLaunchKernelGGL(varlen_empty_finals, dim3(gx, unsigned(nseq)), dim3(256), 0, st, cu, nseq, T, init, fin,
                     per_seq);
  return hipGetLastError();
}

}  // namespace ssd
