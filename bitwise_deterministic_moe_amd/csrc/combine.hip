// Memory-bound reduction kernels around the expert GEMMs.
//
//  gather_combine   out_t = sum over slots j = 0..k-1 (ascending) of
//                   w_tj * rows[slot_row[t*k+j]], float32 accumulation from
//                   0, rounded once.  Forward y (w = topk_prob) and backward
//                   dx (w = 1).  Fixed order: no atomics.
//  scatter_add      atomic-mode counterpart: every row adds w * row into a
//                   zeroed float32 token buffer in arrival order, followed by
//                   cast.
//  dprob_combine    dprob[i] = fixed-shape shuffle tree over the N-tile
//                   partials part[row][0..n_tiles) of row slot_row[i]; 0 for
//                   slots whose expert is not local.  This is the fixed-order
//                   combine of private per-N-tile slots described in the
//                   English digest ("Interpretation") and the French article
//                   ("Optimisation pour le Nemotron ...").
#include "common.h"
#include "kernels.h"

namespace moedet {

template <typename T>
struct Vec;  // 16-byte vectors of the storage type
template <>
struct Vec<uint16_t> {
  static constexpr int N = 8;
  DEV static void load(const uint16_t* p, float (&f)[8]) {
    u32x4_t v = *(const u32x4_t*)p;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      f[2 * w] = bf16_to_f32(v[w] & 0xffffu);
      f[2 * w + 1] = bf16_to_f32(v[w] >> 16);
    }
  }
  DEV static void store(uint16_t* p, const float (&f)[8]) {
    u32x4_t v;
#pragma unroll
    for (int w = 0; w < 4; ++w) v[w] = pack_bf16x2(f[2 * w], f[2 * w + 1]);
    *(u32x4_t*)p = v;
  }
};
template <>
struct Vec<float> {
  static constexpr int N = 4;
  DEV static void load(const float* p, float (&f)[4]) {
    f32x4_t v = *(const f32x4_t*)p;
    f[0] = v[0]; f[1] = v[1]; f[2] = v[2]; f[3] = v[3];
  }
  DEV static void store(float* p, const float (&f)[4]) { *(f32x4_t*)p = f32x4_t{f[0], f[1], f[2], f[3]}; }
};

template <typename T>
__global__ __launch_bounds__(256) void gather_combine_kernel(const T* rows, const int32_t* slot_row,
                                                             const float* weights, int64_t T_, int k,
                                                             int D, T* out, uint64_t seed) {
  constexpr int V = Vec<T>::N;
  const int per_tok = D / V;
  const int64_t units = (T_ * per_tok + 255) / 256;
  const int64_t u = map_unit(blockIdx.x, units, seed);
  if (u < 0) return;
  const int64_t idx = u * 256 + threadIdx.x;
  if (idx >= T_ * per_tok) return;
  const int64_t t = idx / per_tok;
  const int d = (int)(idx % per_tok) * V;
  float acc[V];
#pragma unroll
  for (int q = 0; q < V; ++q) acc[q] = 0.f;
  // slots in groups of 4: the group's row indices, then its rows, are loaded
  // together (one memory round trip each instead of one per slot); they are
  // added in slot order, so the result is the j-ascending sum either way
  constexpr int G = 4;
  for (int j0 = 0; j0 < k; j0 += G) {
    int32_t r[G];
    float w[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      r[i] = j0 + i < k ? slot_row[t * k + j0 + i] : -1;
      w[i] = weights && j0 + i < k ? weights[t * k + j0 + i] : 1.f;
    }
    float f[G][V];
#pragma unroll
    for (int i = 0; i < G; ++i)
      if (r[i] >= 0) Vec<T>::load(rows + (int64_t)r[i] * D + d, f[i]);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (r[i] < 0) continue;
#pragma unroll
      for (int q = 0; q < V; ++q) acc[q] = weights ? __builtin_fmaf(w[i], f[i][q], acc[q]) : acc[q] + f[i][q];
    }
  }
  Vec<T>::store(out + t * D + d, acc);
}

// One wave per (row, segment of 64*V elements); instruction q of the wave
// adds elements q*64 + lane, so every atomic instruction covers 64
// consecutive floats (256 bytes) and every load 64 consecutive elements.
template <typename T>
__global__ __launch_bounds__(256) void scatter_add_kernel(const T* rows, const int32_t* offsets, int el,
                                                          const int32_t* row_tok, const float* row_prob,
                                                          int64_t rows_cap, int D, float* out32,
                                                          uint64_t seed) {
  constexpr int V = sizeof(T) == 2 ? 4 : 1;
  const int per_row = D / (64 * V);
  const int64_t R = offsets[el];
  const int64_t units = (rows_cap * per_row + 3) / 4;
  const int64_t u = map_unit(blockIdx.x, units, seed);
  if (u < 0) return;
  const int lane = threadIdx.x & 63;
  const int64_t wu = u * 4 + (threadIdx.x >> 6);
  if (wu >= R * per_row) return;
  const int64_t r = wu / per_row;
  const int base = (int)(wu % per_row) * 64 * V + lane;
  const float w = row_prob ? row_prob[r] : 1.f;
  const T* src = rows + r * D + base;
  float* o = out32 + (int64_t)row_tok[r] * D + base;
  float f[V];
#pragma unroll
  for (int q = 0; q < V; ++q) {
    if constexpr (sizeof(T) == 2)
      f[q] = bf16_to_f32(src[q * 64]);
    else
      f[q] = src[q * 64];
  }
#pragma unroll
  for (int q = 0; q < V; ++q) atomicAdd(o + q * 64, row_prob ? w * f[q] : f[q]);
}

template <typename T>
__global__ __launch_bounds__(256) void cast_kernel(const float* in, T* out, int64_t n) {
  constexpr int V = Vec<T>::N;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;
  if (i >= n) return;
  float f[V];
#pragma unroll
  for (int q = 0; q < V; ++q) f[q] = in[i + q];
  Vec<T>::store(out + i, f);
}

__global__ __launch_bounds__(256) void zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

// One group of GS = next_pow2(n_tiles) lanes per flat slot; lane q loads
// partial q (or 0 for q >= n_tiles) and the group folds with xor shuffles
// (pairs at distance 1, then 2, 4, ...).  The tree shape depends on n_tiles
// only, and a + b == b + a in IEEE arithmetic, so every lane of the group
// ends with the same bits.
__global__ __launch_bounds__(256) void dprob_combine_kernel(const float* part, const int32_t* slot_row,
                                                            int64_t nslots, int n_tiles, int gs,
                                                            float* dprob, uint64_t seed) {
  const int per_block = 256 / gs;
  const int64_t units = (nslots + per_block - 1) / per_block;
  const int64_t u = map_unit(blockIdx.x, units, seed);
  if (u < 0) return;
  const int q = threadIdx.x % gs;
  const int64_t i = u * per_block + threadIdx.x / gs;
  const bool valid = i < nslots;
  const int32_t r = valid ? slot_row[i] : -1;
  float v = (r >= 0 && q < n_tiles) ? part[(int64_t)r * n_tiles + q] : 0.f;
  for (int d = 1; d < gs; d <<= 1) v = v + __shfl_xor(v, d, 64);
  if (valid && q == 0) dprob[i] = r >= 0 ? v : 0.f;
}

hipError_t launch_gather_combine(const void* rows, const int32_t* slot_row, const float* weights,
                                 int64_t T, int k, int D, void* out, bool bf16, uint64_t seed,
                                 hipStream_t st) {
  const int V = bf16 ? 8 : 4;
  const int64_t units = (T * (D / V) + 255) / 256;
  if (units <= 0) return hipSuccess;
  const int64_t grid = grid_for_units(units);
  if (bf16)
    gather_combine_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)rows, slot_row, weights, T, k,
                                                          D, (uint16_t*)out, seed);
  else
    gather_combine_kernel<float><<<grid, 256, 0, st>>>((const float*)rows, slot_row, weights, T, k, D,
                                                       (float*)out, seed);
  return hipGetLastError();
}

hipError_t launch_scatter_add(const void* rows, const int32_t* offsets, int el, const int32_t* row_tok,
                              const float* row_prob, int64_t rows_cap, int D, float* out32, bool bf16,
                              uint64_t seed, hipStream_t st) {
  const int per_row = D / (64 * (bf16 ? 4 : 1));
  const int64_t units = (rows_cap * per_row + 3) / 4;
  if (units <= 0) return hipSuccess;
  const int64_t grid = grid_for_units(units);
  if (bf16)
    scatter_add_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t*)rows, offsets, el, row_tok, row_prob,
                                                       rows_cap, D, out32, seed);
  else
    scatter_add_kernel<float><<<grid, 256, 0, st>>>((const float*)rows, offsets, el, row_tok, row_prob,
                                                    rows_cap, D, out32, seed);
  return hipGetLastError();
}

hipError_t launch_cast(const float* in32, void* out, int64_t n, bool bf16, hipStream_t st) {
  const int V = bf16 ? 8 : 4;
  const int64_t grid = (n / V + 255) / 256;
  if (grid <= 0) return hipSuccess;
  if (bf16)
    cast_kernel<uint16_t><<<grid, 256, 0, st>>>(in32, (uint16_t*)out, n);
  else
    cast_kernel<float><<<grid, 256, 0, st>>>(in32, (float*)out, n);
  return hipGetLastError();
}

hipError_t launch_zero(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t grid = (n + 255) / 256;
  if (grid > 4096) grid = 4096;
  zero_kernel<<<grid, 256, 0, st>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_dprob_combine(const float* part, const int32_t* slot_row, int64_t nslots, int n_tiles,
                                float* dprob, uint64_t seed, hipStream_t st) {
  int gs = 1;
  while (gs < n_tiles) gs <<= 1;
  const int64_t units = (nslots + 256 / gs - 1) / (256 / gs);
  if (units <= 0) return hipSuccess;
  dprob_combine_kernel<<<grid_for_units(units), 256, 0, st>>>(part, slot_row, nslots, n_tiles, gs, dprob,
                                                              seed);
  return hipGetLastError();
}

}  // namespace moedet
