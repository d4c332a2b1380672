// Throughput probe of the bf16 matrix instruction the attention kernel is
// built on (v_mfma_f32_32x32x16_bf16, 32768 flops each).
//
// Every wave runs `iters` rounds of 8 independent accumulations from
// register operands: no memory traffic, no dependence between consecutive
// instructions of a round, so only the matrix units' issue rate bounds the
// kernel.  Its rate is the practical ceiling that the benchmark reports the
// attention kernel's fraction against, beside the published peak.
#include "common.h"

namespace bsa {

namespace {

constexpr int kChains = 8;

__global__ __launch_bounds__(256) void mfma_peak_kernel(float x, int iters, float *sink) {
  // operands from a kernel argument, so the compiler cannot fold them
  const float xa = x * (float)(threadIdx.x & 7), xb = x + 1.0f;
  const unsigned pa = pack_bf16x2(xa, xb), pb = pack_bf16x2(xb, xa);
  const bf16x8 a = as_bf16x8(u32x4{pa, pb, pa, pb});
  const bf16x8 b = as_bf16x8(u32x4{pb, pa, pb, pa});
  f32x16 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) t += acc[j][e];
  // one lane of the grid stores; the second condition (never true for
  // these operands) makes every lane's sum, and so its chains, live
  if ((blockIdx.x == 0 && threadIdx.x == 0) || t == -1.0f) *sink = t;
}

}  // namespace

long long mfma_peak_flops(int workgroups, int iters) {
  return (long long)workgroups * 4 * iters * kChains * 32768LL;
}

int launch_mfma_peak(int workgroups, int iters, float *sink, hipStream_t stream) {
  clear_pending_error();
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(workgroups), dim3(256), 0, stream, 1.0f / 64, iters,
                     sink);
  return status_of(hipGetLastError());
}

}  // namespace bsa
