// MXFP8 block quantisation: the encoded form (E4M3 values and E8M0 block
// scales) whose bytes the pages fingerprint for low-precision runs (French
// article, section "Méthodologie de débogage du non-déterminisme").  Format
// from the OCP Microscaling Formats (MX) Specification v1.0:
//   block = 32 consecutive elements of a row; shared exponent
//   se = floor(log2(max |v|)) - 8 clamped to [-127, 127] (-127 for a block
//   whose largest magnitude is 0 or a float32 subnormal, where the clamp
//   applies anyway); scale byte se + 127;
//   element code = E4M3 of v * 2^-se, to nearest with ties to even, saturated
//   at 448, sign kept.
// v * 2^-se is exact in float32 whenever it can round to a nonzero code
// (|v * 2^-se| < 512, and values that underflow float32 are far below the
// smallest E4M3 subnormal, 2^-9).  The rounding is the hardware conversion
// on values clamped to +-448 (e4m3x4, equal to the integer rounding
// e4m3_rne); the block maximum is a max of bit patterns, so every output
// byte is exact and independent of execution order.
#include "common.h"
#include "kernels.h"
#include "lowp.h"

namespace moedet {

// Thread: 8 consecutive elements; 4 consecutive threads: one block (the
// blocks of a row are aligned because cols is a multiple of 32).
template <typename T>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const T* in, int64_t rows, int64_t cols, uint8_t* codes,
                                                          uint8_t* scales, uint64_t seed) {
  const int64_t n8 = rows * cols / 8;
  const int64_t u = map_unit(blockIdx.x, (n8 + 255) / 256, seed);
  const int64_t i = (u < 0 ? n8 : u * 256 + threadIdx.x);
  const bool live = i < n8;               // uniform over each 4-thread block
  float v[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = 0.f;
  if (live) load8(in + 8 * i, v);
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) m = max(m, __float_as_uint(v[q]) & 0x7fffffffu);
  m = max(m, (uint32_t)__shfl_xor((int)m, 1));
  m = max(m, (uint32_t)__shfl_xor((int)m, 2));
  const int ef = (int)(m >> 23);
  const int se = ef == 0 ? -127 : min(127, max(-127, ef - 127 - 8));
  const float f = __uint_as_float((uint32_t)(127 - se) << 23);   // 2^-se, exact
  const uint32_t lo = e4m3x4(v[0] * f, v[1] * f, v[2] * f, v[3] * f);
  const uint32_t hi = e4m3x4(v[4] * f, v[5] * f, v[6] * f, v[7] * f);
  if (!live) return;
  *(u32x2_t*)(codes + 8 * i) = u32x2_t{lo, hi};
  if ((threadIdx.x & 3) == 0) scales[(8 * i) / 32] = (uint8_t)(se + 127);
}

// Encode one block of 32 float32 values (the definition above) and store
// its 32 codes (two 16-byte stores) and its scale byte.
DEV void mx_encode_block_store(const float (&v)[32], uint8_t* codes, uint8_t* scale) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = max(m, __float_as_uint(v[i]) & 0x7fffffffu);
  const int ef = (int)(m >> 23);
  const int se = ef == 0 ? -127 : min(127, max(-127, ef - 127 - 8));
  const float f = __uint_as_float((uint32_t)(127 - se) << 23);   // 2^-se, exact
  uint32_t w[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) w[q] = e4m3x4(v[4 * q] * f, v[4 * q + 1] * f, v[4 * q + 2] * f, v[4 * q + 3] * f);
  *(u32x4_t*)codes = u32x4_t{w[0], w[1], w[2], w[3]};
  *(u32x4_t*)(codes + 16) = u32x4_t{w[4], w[5], w[6], w[7]};
  *scale = (uint8_t)(se + 127);
}

// MXFP8 of the transpose of each group's [rows, cols] matrix: a block is 32
// consecutive rows of one column, and the codes of column c are written as
// row c of the output (codes [groups][cols][rows], scales
// [groups][cols][rows/32]).  Same encoding as mx_quantize_kernel.  One thread
// per (column, 32-row block): the 32 loads of a row step are contiguous over
// the wave's 64 columns, and each thread writes its block's 32 codes as two
// 16-byte stores.
template <typename T>
__global__ __launch_bounds__(256) void mx_quantize_t_kernel(const T* in, int64_t groups, int64_t rows, int64_t cols,
                                                            uint8_t* codes, uint8_t* scales, uint64_t seed) {
  const int64_t ncb = (cols + 255) / 256, nrb = rows / 32;
  const int64_t u = map_unit(blockIdx.x, groups * nrb * ncb, seed);
  if (u < 0) return;
  const int64_t g = u / (nrb * ncb), rb = (u / ncb) % nrb, cb = u % ncb;
  const int64_t c = cb * 256 + threadIdx.x;
  if (c >= cols) return;
  const T* src = in + (g * rows + rb * 32) * cols + c;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if constexpr (sizeof(T) == 2)
      v[i] = bf16_to_f32(src[(int64_t)i * cols]);
    else
      v[i] = src[(int64_t)i * cols];
  }
  mx_encode_block_store(v, codes + (g * cols + c) * rows + rb * 32, scales + (g * cols + c) * nrb + rb);
}

// MXFP8 operands of the weight gradients: quantised along the routed rows
// of each expert (the contraction axis of dW1 = X^T dH and dW2 = A^T dY).
// Expert g's rows occupy the padded columns poff[g] .. poff[g+1] of the
// output (its row count rounded up to kMxPad); a block is 32 consecutive
// padded rows of one column, so blocks start at the expert's first row and
// its last block is completed with zeros.  Padded row j of expert g is
// routed row offsets[g] + (j - poff[g]) while below its count, and reads
//   token: src[row_tok[r]] (x or dY, gathered by token),
//   row:   src[r] (dH),
//   act_p: p_r * (relu(h_r))^2 from h = src[r], relu(v) = v > 0 ? v : +0,
//          the square rounded to float32 and then the product.
// Same encoding as mx_quantize_t_kernel.  Codes and scales are stored
// slice-major, [rpad / 64][cols][64] and [rpad / 64][cols][2]: the 64 codes
// (and two scales) of one column and 64-row slice, columns side by side, so
// that the weight-gradient GEMM reads a tile's slice as one contiguous run
// and this kernel writes whole runs.  Blocks at or past poff[el] are not
// written.
//
// Workgroup: 128 padded rows (two slices) by 256 columns, in four chunks of
// 64.  The padded and routed row offsets are copied to LDS once (one memory
// round trip) and each of the 128 rows finds its expert by binary search
// there, then its source row (and p) once; per chunk the rows are loaded 16
// bytes a lane (eight lanes a row) into LDS as float32 and thread (column,
// block) encodes its 32 values: a wave stores two contiguous 1 KiB runs of
// codes (16 columns of each slice).
constexpr int kQwRows = 128, kQwCols = 64, kQwChunks = 4;
template <int KIND>
__global__ __launch_bounds__(256) void mx_quantize_wgrad_kernel(MxWgradQuantParams P) {
  __shared__ float s_v[kQwRows][kQwCols + 1];
  __shared__ int s_poff[kMaxExperts + 1];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int64_t s_src[kQwRows];   // source row of each tile row, -1: padding
  __shared__ float s_p[kQwRows];
  const int64_t ncb = P.cols / (kQwCols * kQwChunks), nrb = (P.rpad + kQwRows - 1) / kQwRows;
  const int64_t u = map_unit(blockIdx.x, nrb * ncb, P.seed);
  if (u < 0) return;
  const int j0 = (int)((u / ncb) * kQwRows);
  const int64_t cbase = (u % ncb) * (kQwCols * kQwChunks);
  const int total = P.poff[P.el];
  if (j0 >= total) return;
  const int tid = threadIdx.x;
  for (int g = tid; g <= P.el; g += 256) {
    s_poff[g] = P.poff[g];
    s_off[g] = P.offsets[g];
  }
  __syncthreads();
  if (tid < kQwRows) {
    // routed row of padded row j (padding: none), its expert being the last
    // g with poff[g] <= j
    const int j = j0 + tid;
    int64_t src = -1;
    float p = 0.f;
    if (j < total) {
      int lo = 0, hi = P.el - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_poff[mid] <= j) lo = mid; else hi = mid - 1;
      }
      const int local = j - s_poff[lo];
      if (local < s_off[lo + 1] - s_off[lo]) {
        const int r = s_off[lo] + local;
        src = KIND == kMxwToken ? (int64_t)P.row_tok[r] : (int64_t)r;
        if constexpr (KIND == kMxwActP) p = P.row_prob[r];
      }
    }
    s_src[tid] = src;
    s_p[tid] = p;
  }
  __syncthreads();
  const int cc = (tid & 7) * 8;   // this lane's 8 columns of a row
  const int c = tid >> 2, b = tid & 3;
  const int jb = j0 + 32 * b;
  // every chunk's loads issued up front: 4 rows x 16 bytes per chunk a lane
  constexpr int kPass = kQwRows / 32;
  u32x4_t raw[kQwChunks][kPass];
#pragma unroll
  for (int chunk = 0; chunk < kQwChunks; ++chunk)
#pragma unroll
    for (int pass = 0; pass < kPass; ++pass) {
      const int64_t srow = s_src[pass * 32 + (tid >> 3)];
      raw[chunk][pass] = srow >= 0 ? *(const u32x4_t*)(P.src + srow * P.cols + cbase + chunk * kQwCols + cc)
                                   : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
  for (int chunk = 0; chunk < kQwChunks; ++chunk) {
    const int64_t c0 = cbase + chunk * kQwCols;
#pragma unroll
    for (int pass = 0; pass < kPass; ++pass) {
      const int i = pass * 32 + (tid >> 3);
      float v[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        v[2 * w] = bf16_to_f32(raw[chunk][pass][w] & 0xffffu);
        v[2 * w + 1] = bf16_to_f32(raw[chunk][pass][w] >> 16);
      }
      if constexpr (KIND == kMxwActP) {
        // padding rows hold zeros (p = 0 there), which stay +0
        const float pr = s_p[i];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float rl = v[q] > 0.f ? v[q] : 0.f;
          const float sq = rl * rl;
          v[q] = pr * sq;
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) s_v[i][cc + q] = v[q];
    }
    __syncthreads();
    if (jb < total) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = s_v[32 * b + i][c];
      const int64_t at = ((int64_t)(jb / 64) * P.cols + c0 + c) * 2 + ((jb / 32) & 1);   // (slice, column, block)
      mx_encode_block_store(v, P.codes + at * 32, P.scales + at);
    }
    __syncthreads();
  }
}

hipError_t launch_mx_quantize_wgrad(const MxWgradQuantParams& P, hipStream_t st) {
  const int64_t units = ((P.rpad + kQwRows - 1) / kQwRows) * (P.cols / (kQwCols * kQwChunks));
  if (units == 0) return hipSuccess;
  const int64_t grid = grid_for_units(units);
  if (P.kind == kMxwToken)
    mx_quantize_wgrad_kernel<kMxwToken><<<grid, 256, 0, st>>>(P);
  else if (P.kind == kMxwRow)
    mx_quantize_wgrad_kernel<kMxwRow><<<grid, 256, 0, st>>>(P);
  else
    mx_quantize_wgrad_kernel<kMxwActP><<<grid, 256, 0, st>>>(P);
  return hipGetLastError();
}

hipError_t launch_mx_quantize_t(const void* in, bool bf16, int64_t groups, int64_t rows, int64_t cols,
                                uint8_t* codes, uint8_t* scales, uint64_t seed, hipStream_t st) {
  const int64_t units = groups * (rows / 32) * ((cols + 255) / 256);
  if (units == 0) return hipSuccess;
  const int64_t grid = grid_for_units(units);
  if (bf16)
    mx_quantize_t_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)in, groups, rows, cols, codes, scales,
                                                         seed);
  else
    mx_quantize_t_kernel<float><<<grid, 256, 0, st>>>((const float*)in, groups, rows, cols, codes, scales, seed);
  return hipGetLastError();
}

hipError_t launch_mx_quantize(const void* in, bool bf16, int64_t rows, int64_t cols, uint8_t* codes,
                              uint8_t* scales, uint64_t seed, hipStream_t st) {
  const int64_t n8 = rows * cols / 8;
  if (n8 == 0) return hipSuccess;
  const int64_t grid = grid_for_units((n8 + 255) / 256);
  if (bf16)
    mx_quantize_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)in, rows, cols, codes, scales, seed);
  else
    mx_quantize_kernel<float><<<grid, 256, 0, st>>>((const float*)in, rows, cols, codes, scales, seed);
  return hipGetLastError();
}

}  // namespace moedet
