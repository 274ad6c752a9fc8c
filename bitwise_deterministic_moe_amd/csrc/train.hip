// The two pieces a deterministic train step of the layer needs besides the
// forward and backward ("Trillion-Parameter Pretraining Goes
// Bitwise-Deterministic", section "Interpretation": a full-precision source of
// truth, and the runtime representation reconstructed through the same
// conversion path used in training):
//   router forward: logits[t, e] = sum over d ascending of x[t, d] * wr[e, d],
//                   float32 fused multiply-adds (one thread per logit);
//   SGD step:       master[i] = master[i] - lr * grad[i] (float32, one fused
//                   multiply-add), runtime[i] = master[i] rounded to the
//                   storage type (round-to-nearest-even).
// Neither has a reduction across threads, so both are bit-exact by
// construction.
#include "common.h"
#include "kernels.h"

namespace moedet {

DEV void dot_load8(const uint16_t* p, float (&f)[8]) {
  const u32x4_t v = *(const u32x4_t*)p;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f[2 * w] = bf16_to_f32(v[w] & 0xffffu);
    f[2 * w + 1] = bf16_to_f32(v[w] >> 16);
  }
}
DEV void dot_load8(const float* p, float (&f)[8]) {
  const f32x4_t a = *(const f32x4_t*)p, b = *(const f32x4_t*)(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = a[i];
    f[4 + i] = b[i];
  }
}

// Thread (t, e); consecutive threads take consecutive experts of one token,
// so a wave shares the token's row and reads 64 router rows.
template <typename T>
__global__ __launch_bounds__(256) void router_fwd_kernel(const T* x, const T* wr, int64_t tokens, int E, int D,
                                                         float* logits, uint64_t seed) {
  const int64_t units = (tokens * E + 255) / 256;
  const int64_t u = map_unit(blockIdx.x, units, seed);
  if (u < 0) return;
  const int64_t idx = u * 256 + threadIdx.x;
  if (idx >= tokens * E) return;
  const int64_t t = idx / E;
  const int e = (int)(idx % E);
  const T* xr = x + t * D;
  const T* wrow = wr + (int64_t)e * D;
  float acc = 0.f;
  for (int d = 0; d < D; d += 8) {
    float a[8], b[8];
    dot_load8(xr + d, a);
    dot_load8(wrow + d, b);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(a[i], b[i], acc);
  }
  logits[idx] = acc;
}

template <typename T>
__global__ __launch_bounds__(256) void sgd_kernel(float* master, const float* grad, int64_t n, float lr, T* runtime) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float m = __builtin_fmaf(-lr, grad[i], master[i]);
  master[i] = m;
  if constexpr (sizeof(T) == 2)
    runtime[i] = (uint16_t)f32_to_bf16(m);
  else
    runtime[i] = m;
}

hipError_t launch_router_fwd(const void* x, const void* wr, int64_t T, int E, int D, float* logits, bool bf16,
                             uint64_t seed, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int64_t grid = grid_for_units((T * E + 255) / 256);
  if (bf16)
    router_fwd_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)x, (const uint16_t*)wr, T, E, D, logits, seed);
  else
    router_fwd_kernel<float><<<grid, 256, 0, st>>>((const float*)x, (const float*)wr, T, E, D, logits, seed);
  return hipGetLastError();
}

hipError_t launch_sgd(float* master, const float* grad, int64_t n, float lr, void* runtime, bool bf16,
                      hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t grid = (n + 255) / 256;
  if (bf16)
    sgd_kernel<uint16_t><<<grid, 256, 0, st>>>(master, grad, n, lr, (uint16_t*)runtime);
  else
    sgd_kernel<float><<<grid, 256, 0, st>>>(master, grad, n, lr, (float*)runtime);
  return hipGetLastError();
}

}  // namespace moedet
