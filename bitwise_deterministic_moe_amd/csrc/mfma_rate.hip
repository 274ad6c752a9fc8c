// Attainable bf16 MFMA rate of the device: a loop of independent
// v_mfma_f32_32x32x16_bf16 on register operands, with no memory traffic in
// the loop, so that a timed launch measures the matrix cores alone (at the
// shader clock the device holds under that load).  The GEMM kernels' rates
// are quoted against both this figure and the nominal dense peak.
#include "common.h"
#include "kernels.h"

namespace moedet {

// Every wave issues iters x 8 MFMAs into 8 independent accumulators (128
// registers; eight MFMAs of 32 clocks between dependent ones hide the MFMA
// latency).  Both operands hold the value v in every element, so each MFMA
// adds 16 v^2 to every accumulator element; thread t of block b writes the
// sum of its 128 accumulator elements to sink[256 b + t], which keeps the
// work live and lets a caller check it (exactly 2048 v^2 iters while that is
// exact in float32).
__global__ __launch_bounds__(256) void mfma_rate_kernel(int64_t iters, float v, float* sink) {
  const uint16_t bits = (uint16_t)(__float_as_uint(v) >> 16);  // v must be bf16-representable
  const uint32_t w = (uint32_t)bits * 0x10001u;
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, u32x4_t{w, w, w, w});
  f32x16_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
#pragma unroll 1
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

hipError_t launch_mfma_rate(int64_t blocks, int64_t iters, float v, float* sink, hipStream_t st) {
  mfma_rate_kernel<<<blocks, 256, 0, st>>>(iters, v, sink);
  return hipGetLastError();
}

}  // namespace moedet
