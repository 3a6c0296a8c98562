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
// Work-group: one (batch, chunk) and KH heads of one B/C group, 4 waves. The
// token axis is the contraction axis, but x and B are stored token-major, so
// each 32-token slice is transposed on its way into LDS (8 x 8 bf16 blocks
// transposed in registers, W scaled in fp32 before its single bf16 rounding).
// The B^T slice is shared by the KH heads. Each wave owns KH*(P/32)*(N/32)/4
// output tiles of 32 x 32 (fp32 accumulators) and reads its operands from LDS
// with 16-byte loads; row stride 40 bf16 (80 B) keeps 16 lanes on distinct
// banks. Output tiles go to HBM as fp32 rows of 32 consecutive n.
#include "mfma_util.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kSK = 32;          // tokens per contraction slice
constexpr int kRS = kSK + 8;     // LDS row stride (bf16 elements)
constexpr int kMaxQ = 256;

template <int N, int P, int KH>
__global__ __launch_bounds__(kThreads) void chunk_state_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const float* __restrict__ Acs,
    const float* __restrict__ dtq, float* __restrict__ S, int T, int H, int G, int Q, int nc,
    int nhg) {
  __shared__ __attribute__((aligned(16))) uint16_t sBt[N][kRS];
  __shared__ __attribute__((aligned(16))) uint16_t sWt[KH][P][kRS];
  __shared__ float sw[KH][kMaxQ];

  constexpr int NT = N / 32, PT = P / 32;
  constexpr int TILES = KH * PT * NT;
  constexpr int TPW = (TILES + 3) / 4;
  const int id = xcd_swizzle(blockIdx.x, gridDim.x);
  const int hg = id % nhg;
  const int bc = id / nhg;
  const int c = bc % nc, b = bc / nc;
  const int h0 = hg * KH;
  const int g = h0 / (H / G);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g2 = lane >> 5;
  const long t0 = long(c) * Q;

  // w_s = exp(Acs_{Q-1} - Acs_s) * dt_s for the whole chunk, per head
  for (int e = tid; e < KH * Q; e += kThreads) {
    const int kh = e / Q, i = e % Q;
    const size_t arow = ((size_t(b) * H + h0 + kh) * nc + c) * Q;
    sw[kh][i] = exp_fast(Acs[arow + Q - 1] - Acs[arow + i]) * dtq[arow + i];
  }

  f32x16 acc[TPW];
#pragma unroll
  for (int m = 0; m < TPW; ++m) acc[m] = zero16();

  constexpr int NBB = (kSK / 8) * (N / 8);        // 8x8 blocks of the B slice
  constexpr int NWB = KH * (kSK / 8) * (P / 8);   // 8x8 blocks of the W slices

  for (int s0 = 0; s0 < Q; s0 += kSK) {
    __syncthreads();  // sw written / previous slice consumed
    for (int blk = tid; blk < NBB + NWB; blk += kThreads) {
      u32x4 in[8], out[8];
      if (blk < NBB) {
        const int tg = blk / (N / 8), ng = blk % (N / 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const long t = t0 + s0 + 8 * tg + i;
          const long tc = t < T ? t : T - 1;
          in[i] = keep_or_zero(t < T, load16(Bm + ((size_t(b) * T + tc) * G + g) * N + 8 * ng));
        }
        transpose8x8_b16(in, out);
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(&sBt[8 * ng + j][8 * tg]) = out[j];
      } else {
        const int wb = blk - NBB;
        const int kh = wb / ((kSK / 8) * (P / 8));
        const int r = wb % ((kSK / 8) * (P / 8));
        const int tg = r / (P / 8), pg = r % (P / 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const long t = t0 + s0 + 8 * tg + i;
          const long tc = t < T ? t : T - 1;
          const u32x4 raw =
              keep_or_zero(t < T, load16(x + ((size_t(b) * T + tc) * H + h0 + kh) * P + 8 * pg));
          const float w = sw[kh][s0 + 8 * tg + i];
#pragma unroll
          for (int m = 0; m < 4; ++m) in[i][m] = pack_bf16x2(bf16_lo(raw[m]) * w, bf16_hi(raw[m]) * w);
        }
        transpose8x8_b16(in, out);
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(&sWt[kh][8 * pg + j][8 * tg]) = out[j];
      }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int tile = wave + 4 * m;
      if (tile < TILES) {
        const int kh = tile / (PT * NT);
        const int r = tile % (PT * NT);
        const int pb = r / NT, nb = r % NT;
#pragma unroll
        for (int kk = 0; kk < kSK / 16; ++kk) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(&sWt[kh][32 * pb + l32][16 * kk + 8 * g2]);
          const u32x4 bb = *reinterpret_cast<const u32x4*>(&sBt[32 * nb + l32][16 * kk + 8 * g2]);
          acc[m] = mfma32x32x16(a, bb, acc[m]);
        }
      }
    }
  }

#pragma unroll
  for (int m = 0; m < TPW; ++m) {
    const int tile = wave + 4 * m;
    if (tile < TILES) {
      const int kh = tile / (PT * NT);
      const int r = tile % (PT * NT);
      const int pb = r / NT, nb = r % NT;
      float* out = S + ((size_t(b) * nc + c) * H + h0 + kh) * size_t(P) * N;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int p = 32 * pb + 8 * (q / 4) + 4 * g2 + (q % 4);
        out[size_t(p) * N + 32 * nb + l32] = acc[m][q];
      }
    }
  }
}

template <int N, int P, int KH>
hipError_t launch_t(const FwdShape& s, const void* x, const void* B, const float* Acs,
                    const float* dtq, float* S, hipStream_t st) {
  const int nhg = s.H / KH;
  const long blocks = long(s.b) * s.nc * nhg;
  hipLaunchKernelGGL((chunk_state_mfma_kernel<N, P, KH>), dim3(unsigned(blocks)), dim3(kThreads), 0,
                     st, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(B), Acs, dtq, S,
                     s.T, s.H, s.G, s.Q, s.nc, nhg);
  return hipGetLastError();
}

template <int N, int P>
hipError_t launch_np(const FwdShape& s, const void* x, const void* B, const float* Acs,
                     const float* dtq, float* S, hipStream_t st) {
  // two heads per work-group share the staged B slice, while the fp32
  // accumulators stay within 128 registers per lane
  if constexpr ((P / 32) * (N / 32) * 2 <= 32) {
    if ((s.H / s.G) % 2 == 0) return launch_t<N, P, 2>(s, x, B, Acs, dtq, S, st);
  }
  return launch_t<N, P, 1>(s, x, B, Acs, dtq, S, st);
}

template <int N>
hipError_t launch_n(const FwdShape& s, const void* x, const void* B, const float* Acs,
                    const float* dtq, float* S, hipStream_t st) {
  switch (s.P) {
    case 32: return launch_np<N, 32>(s, x, B, Acs, dtq, S, st);
    case 64: return launch_np<N, 64>(s, x, B, Acs, dtq, S, st);
    case 128: return launch_np<N, 128>(s, x, B, Acs, dtq, S, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_state_mfma(const FwdShape& s, const void* x, const void* B,
                                   const float* Acs, const float* dtq, float* S, hipStream_t st) {
  switch (s.N) {
    case 32: return launch_n<32>(s, x, B, Acs, dtq, S, st);
    case 64: return launch_n<64>(s, x, B, Acs, dtq, S, st);
    case 128: return launch_n<128>(s, x, B, Acs, dtq, S, st);
    case 256: return launch_n<256>(s, x, B, Acs, dtq, S, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace ssd
