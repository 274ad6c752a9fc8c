// NVFP4 block quantisation: E2M1 element codes, an E4M3 scale per 16
// consecutive elements of a row and a float32 scale for the whole tensor, the
// second low-precision form whose encoded values and scale buffers the pages
// fingerprint (French article, section "Méthodologie de débogage du
// non-déterminisme").  The pages do not define the format; this follows
// NVIDIA's public description of NVFP4, with every decision taken in these
// float32 steps:
//   g = amax / 2688 (= 6 * 448; 1 if that is 0)   tensor scale
//   x = amax_block / (6 g)  ->  block scale code sb = E4M3(x)
//   d = value(sb) * g       ->  element code = E2M1(|v| / d) (0 if d == 0),
//                               sign kept
// E4M3 and E2M1 round to nearest with ties to the even code and saturate at
// 448 and 6.  Two element codes share a byte, the even element in the low
// nibble.  Three launches: the tensor amax (a max of |v| bit patterns, so its
// atomics give the same word in any order), g from it (one thread), then the
// codes.
#include "common.h"
#include "kernels.h"
#include "lowp.h"

namespace moedet {

// E2M1 code of |y| (y >= 0): 0, 0.5, 1, 1.5, 2, 3, 4, 6; see the header comment.
DEV uint32_t e2m1_rne(float y) {
  const uint32_t a = __float_as_uint(y);
  if (a >= 0x40c00000u) return 7u;                                   // >= 6
  if (a >= 0x3f800000u) return ((a + 0x1fffffu + ((a >> 22) & 1u)) >> 22) - 252u;   // [1, 6): 1 mantissa bit
  return (uint32_t)__builtin_rintf(y * 2.0f);                        // [0, 1): steps of 0.5
}

// value of an E4M3 code (finite codes only)
DEV float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e == 0 ? (float)m * 0x1p-9f : (float)(8u + m) * __uint_as_float((e + 117u) << 23);   // (8+m) 2^(e-10)
}

// Grid-stride over 8-element groups; the workgroup's max (waves, then LDS)
// goes to the word with one atomic per workgroup, so at most kAmaxBlocks
// atomics meet at one address.
constexpr int kAmaxBlocks = 1024;
template <typename T>
__global__ __launch_bounds__(256) void nvfp4_amax_kernel(const T* in, int64_t n8, uint32_t* amax_bits) {
  __shared__ uint32_t s_m[4];
  uint32_t m = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    float v[8];
    load8(in + 8 * i, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) m = max(m, __float_as_uint(v[q]) & 0x7fffffffu);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  if ((threadIdx.x & 63) == 0) s_m[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(s_m[0], s_m[1]), max(s_m[2], s_m[3]));
    if (m != 0) atomicMax(amax_bits, m);
  }
}

__global__ void nvfp4_tensor_scale_kernel(float* g) {
  const float amax = __uint_as_float(*(const uint32_t*)g);
  const float s = amax / 2688.0f;
  *g = s > 0.f ? s : 1.0f;
}

// Thread: 8 consecutive elements; 2 consecutive threads: one block (blocks of
// a row are aligned because cols is a multiple of 16).
template <typename T>
__global__ __launch_bounds__(256) void nvfp4_quantize_kernel(const T* in, int64_t n8, const float* gp, uint8_t* codes,
                                                             uint8_t* scales, uint64_t seed) {
  const int64_t u = map_unit(blockIdx.x, (n8 + 255) / 256, seed);
  const int64_t i = (u < 0 ? n8 : u * 256 + threadIdx.x);
  const bool live = i < n8;               // uniform over each 2-thread block
  float v[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = 0.f;
  if (live) load8(in + 8 * i, v);
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) m = max(m, __float_as_uint(v[q]) & 0x7fffffffu);
  m = max(m, (uint32_t)__shfl_xor((int)m, 1));
  const float g = *gp;
  const float t = 6.0f * g;
  const uint32_t sb = e4m3_rne(__uint_as_float(m) / t);
  const float d = e4m3_value(sb) * g;
  uint32_t packed = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t c = d != 0.f ? e2m1_rne(__builtin_fabsf(v[q]) / d) : 0u;
    packed |= (c | ((__float_as_uint(v[q]) >> 28) & 0x8u)) << (4 * q);
  }
  if (!live) return;
  *(uint32_t*)(codes + 4 * i) = packed;
  if ((threadIdx.x & 1) == 0) scales[i / 2] = (uint8_t)sb;
}

hipError_t launch_nvfp4_quantize(const void* in, bool bf16, int64_t rows, int64_t cols, uint8_t* codes,
                                 uint8_t* scales, float* global_scale, uint64_t seed, hipStream_t st) {
  const int64_t n8 = rows * cols / 8;
  hipError_t e = launch_zero(global_scale, 1, st);
  if (e != hipSuccess) return e;
  const int64_t grid = grid_for_units((n8 + 255) / 256);
  if (n8 > 0) {
    const int64_t ag = grid < kAmaxBlocks ? grid : kAmaxBlocks;
    if (bf16)
      nvfp4_amax_kernel<uint16_t><<<ag, 256, 0, st>>>((const uint16_t*)in, n8, (uint32_t*)global_scale);
    else
      nvfp4_amax_kernel<float><<<ag, 256, 0, st>>>((const float*)in, n8, (uint32_t*)global_scale);
  }
  nvfp4_tensor_scale_kernel<<<1, 1, 0, st>>>(global_scale);
  if (n8 > 0) {
    if (bf16)
      nvfp4_quantize_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)in, n8, global_scale, codes, scales, seed);
    else
      nvfp4_quantize_kernel<float><<<grid, 256, 0, st>>>((const float*)in, n8, global_scale, codes, scales, seed);
  }
  return hipGetLastError();
}

}  // namespace moedet
