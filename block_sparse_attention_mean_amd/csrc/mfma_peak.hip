// Throughput probe of the bf16 matrix instruction the attention kernel is
// built on (v_mfma_f32_32x32x16_bf16, 32768 flops each).
//
// Every wave runs `iters` rounds of 8 independent accumulations from
// register operands: no memory traffic, no dependence between consecutive
// instructions of a round, so only the matrix units bound the kernel.  What
// they sustain depends on the operand data as well as on the instruction
// count: the chip lowers its clock under the power of toggling operands.
// Two operand modes:
//   random       three sets of random bf16 operands (random sign, exponent
//                spanning [1/4, 4), random mantissa; a per-lane hash of
//                the seed and register index), consecutive instructions
//                taking different sets, as the attention kernel's gathered
//                keys do;
//   low entropy  the same small operands for every instruction of a lane
//                (a few distinct values with short mantissas), the most
//                favourable case.
// The random mode is the practical peak the benchmark states the attention
// kernel's fraction against, beside the published one.
#include "common.h"

namespace bsa {

namespace {

constexpr int kChains = 8;
constexpr int kSets = 3;

// Two bf16 values with random sign, exponent 2^-2 .. 2^1 and mantissa, from
// a hash of (lane, register index); each register's value is independent,
// so generating them keeps few registers live.
__device__ __forceinline__ unsigned random_bf16x2(unsigned lane, unsigned idx, unsigned seed) {
  unsigned v = (lane * 0x9e3779b1u) ^ (idx * 0x85ebca77u) ^ seed;
  v ^= v >> 15;
  v *= 0x2c1b3c6du;
  v ^= v >> 12;
  v *= 0x297a2d39u;
  v ^= v >> 15;
  const unsigned m = 0x80ff80ffu & (v ^ (v >> 7));          // signs and mantissas
  const unsigned e = ((v >> 5) & 0x00030003u) + 0x007d007du;  // exponents 125 .. 128
  return (m & 0x807f807fu) | (e << 7);
}

template <int MODE>
__global__ __launch_bounds__(256) void mfma_peak_kernel(unsigned seed, int iters, float *sink) {
  bf16x8 a[kSets], b[kSets];
  if (MODE == 0) {
    const unsigned lane = blockIdx.x * 256u + threadIdx.x;
#pragma unroll
    for (int t = 0; t < kSets; ++t) {
      u32x4 ua, ub;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ua[e] = random_bf16x2(lane, 8 * t + e, seed);
        ub[e] = random_bf16x2(lane, 8 * t + 4 + e, seed);
      }
      a[t] = as_bf16x8(ua);
      b[t] = as_bf16x8(ub);
    }
  } else {
    // operands from a kernel argument, so the compiler cannot fold them
    const float x = __builtin_bit_cast(float, 0x3c800000u + (seed & 0xffu));  // ~1/64
    const float xa = x * (float)(threadIdx.x & 7), xb = x + 1.0f;
    const unsigned pa = pack_bf16x2(xa, xb), pb = pack_bf16x2(xb, xa);
#pragma unroll
    for (int t = 0; t < kSets; ++t) {
      a[t] = as_bf16x8(u32x4{pa, pb, pa, pb});
      b[t] = as_bf16x8(u32x4{pb, pa, pb, pa});
    }
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j % kSets], b[j % kSets], acc[j], 0, 0, 0);
  }
  // one element per chain keeps every instruction live (each writes all 16
  // elements); reading all of them would take 128 more registers and lower
  // the waves a SIMD can hold
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) t += acc[j][j];
  // one lane of the grid stores; the second condition (never true for
  // these operands) makes every lane's sum, and so its chains, live
  if ((blockIdx.x == 0 && threadIdx.x == 0) || t == -1.0f) *sink = t;
}

}  // namespace

long long mfma_peak_flops(int workgroups, int iters) {
  return (long long)workgroups * 4 * iters * kChains * 32768LL;
}

int launch_mfma_peak(int workgroups, int iters, int operands, float *sink, hipStream_t stream) {
  clear_pending_error();
  if (operands == 0)
    hipLaunchKernelGGL(mfma_peak_kernel<0>, dim3(workgroups), dim3(256), 0, stream, 12345u, iters,
                       sink);
  else
    hipLaunchKernelGGL(mfma_peak_kernel<1>, dim3(workgroups), dim3(256), 0, stream, 0u, iters, sink);
  return status_of(hipGetLastError());
}

}  // namespace bsa
