// Chunk-wise tensor fingerprint (the French article, section "Méthodologie
// de débogage du non-déterminisme": GPU fingerprints recording shape, dtype
// and element count, chunk-wise for order-sensitive data).
//
//   v_i = mix64(bits_i ^ (i * GAMMA))          per element, bits zero-extended
//   H_c = mix64((sum_{i in chunk c} v_i) ^ c)  sum mod 2^64
//   total: h = GAMMA, h = mix64(h ^ w) for w in [dtype, ndim, shape..., numel,
//          chunk, H_0, ..., H_{m-1}]
//
// Wrapping integer addition is associative and commutative, so the order in
// which the workgroup adds the v_i cannot change H_c; all arithmetic is
// integer, hence bit-exact.
#include "common.h"
#include "kernels.h"

namespace moedet {

struct FoldWords {
  uint64_t w[16];
  int n;
};

template <int W>
DEV uint64_t load_bits(const void* p, int64_t i) {
  if constexpr (W == 1) return ((const uint8_t*)p)[i];
  if constexpr (W == 2) return ((const uint16_t*)p)[i];
  if constexpr (W == 4) return ((const uint32_t*)p)[i];
  return ((const uint64_t*)p)[i];
}

template <int W>
DEV uint64_t word_bits(const u32x4_t& q, int e) {
  if constexpr (W == 1) return (q[e >> 2] >> (8 * (e & 3))) & 0xffu;
  if constexpr (W == 2) return (q[e >> 1] >> (16 * (e & 1))) & 0xffffu;
  if constexpr (W == 4) return q[e];
  return ((uint64_t)q[2 * e + 1] << 32) | q[2 * e];
}

// One workgroup per chunk.  When the chunk starts on a 16-byte boundary
// (vec), each thread reads 16-byte words (16/W elements, streamed past the
// caches) and the chunk's last partial word element by element; the terms
// and their wrapping sum are the same either way.
template <int W>
__global__ __launch_bounds__(256) void fp_chunk_kernel(const void* data, int64_t n, int64_t chunk, int vec,
                                                       uint64_t* hashes) {
  __shared__ uint64_t s_red[4];
  const int64_t c = blockIdx.x;
  const int64_t lo = c * chunk, hi = min(n, lo + chunk);
  uint64_t acc = 0;
  int64_t tail = lo;
  if (vec) {
    constexpr int V = 16 / W;
    const int64_t nv = (hi - lo) / V;
    const u32x4_t* p = (const u32x4_t*)((const char*)data + lo * W);
    for (int64_t v = threadIdx.x; v < nv; v += 256) {
      const u32x4_t q = __builtin_nontemporal_load(p + v);
      const uint64_t i0 = (uint64_t)(lo + v * V);
#pragma unroll
      for (int e = 0; e < V; ++e) acc += mix64(word_bits<W>(q, e) ^ ((i0 + e) * kGamma));
    }
    tail = lo + nv * V;
  }
  for (int64_t i = tail + threadIdx.x; i < hi; i += 256) acc += mix64(load_bits<W>(data, i) ^ ((uint64_t)i * kGamma));
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) hashes[c] = mix64((s_red[0] + s_red[1] + s_red[2] + s_red[3]) ^ (uint64_t)c);
}

// The ordered fold by one wave: 64 chunk hashes are loaded at a time (the
// next 64 while these are folded) and folded in index order from lane
// reads, so the sequential chain waits on no memory access.
__global__ __launch_bounds__(64) void fp_fold_kernel(FoldWords head, const uint64_t* hashes, int64_t m,
                                                     uint64_t* total) {
  const int lane = threadIdx.x;
  uint64_t h = kGamma;
  for (int i = 0; i < head.n; ++i) h = mix64(h ^ head.w[i]);
  uint64_t nxt = lane < m ? hashes[lane] : 0;
  for (int64_t b = 0; b < m; b += 64) {
    const uint64_t cur = nxt;
    nxt = b + 64 + lane < m ? hashes[b + 64 + lane] : 0;
    const int cnt = (int)min((int64_t)64, m - b);
    const uint32_t lo32 = (uint32_t)cur, hi32 = (uint32_t)(cur >> 32);
    for (int j = 0; j < cnt; ++j) {
      const uint64_t v = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi32, j) << 32) |
                         (uint32_t)__builtin_amdgcn_readlane((int)lo32, j);
      h = mix64(h ^ v);
    }
  }
  if (lane == 0) *total = h;
}

hipError_t launch_fingerprint(const void* data, int width, int64_t n, int64_t chunk, const uint64_t* words,
                              int nwords, uint64_t* chunk_hashes, uint64_t* total, hipStream_t st) {
  FoldWords head{};
  if (nwords > 16) return hipErrorInvalidValue;
  for (int i = 0; i < nwords; ++i) head.w[i] = words[i];
  head.n = nwords;
  const int64_t m = (n + chunk - 1) / chunk;
  // 16-byte reads when every chunk starts on a 16-byte boundary
  const int vec = ((uintptr_t)data % 16 == 0) && ((chunk * width) % 16 == 0);
  if (m > 0) {
    switch (width) {
      case 1: fp_chunk_kernel<1><<<m, 256, 0, st>>>(data, n, chunk, vec, chunk_hashes); break;
      case 2: fp_chunk_kernel<2><<<m, 256, 0, st>>>(data, n, chunk, vec, chunk_hashes); break;
      case 4: fp_chunk_kernel<4><<<m, 256, 0, st>>>(data, n, chunk, vec, chunk_hashes); break;
      case 8: fp_chunk_kernel<8><<<m, 256, 0, st>>>(data, n, chunk, vec, chunk_hashes); break;
      default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  fp_fold_kernel<<<1, 64, 0, st>>>(head, chunk_hashes, m, total);
  return hipGetLastError();
}

}  // namespace moedet
