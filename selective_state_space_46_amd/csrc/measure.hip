// measure.hip -- the bf16 matrix-core rate probe (ssd_measure.h).
#include "mfma_util.h"
#include "ssd_measure.h"

namespace ssd {
namespace {

// 8 independent accumulator chains per wave keep the matrix pipe busy between
// dependent instructions; the operands vary by lane so no result is constant.
__global__ __launch_bounds__(256) void mfma_bf16_probe_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  const u32x4 a = u32x4{0x3f803f80u + lane, 0x3f003f00u, 0x3e803e80u, 0x3f403f40u};
  const u32x4 b = u32x4{0x3c003c00u, 0x3c803c80u + lane, 0x3b803b80u, 0x3c403c40u};
  f32x16 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = zero16();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = mfma32x32x16(a, b, acc[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  out[size_t(blockIdx.x) * 256 + threadIdx.x] = s;
}

}  // namespace
}  // namespace ssd

extern "C" ssd_status ssd_mfma_bf16_probe(int workgroups, int iters, float* out, void* stream) {
  if (workgroups < 1 || iters < 1) return SSD_ERR_SHAPE;
  if (double(workgroups) * 4.0 * iters * 8.0 * 32768.0 > 4.6e18) return SSD_ERR_SHAPE;
  if (!out) return SSD_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(out) & 15u) return SSD_ERR_ALIGN;
  hipLaunchKernelGGL(ssd::mfma_bf16_probe_kernel, dim3(unsigned(workgroups)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? SSD_OK : SSD_ERR_HIP;
}
