// Device helpers shared by the gfx950 kernels of libmoedet.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define DEV __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

namespace moedet {

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator dies, workgroups dealt round-robin

// ------------------------------------------------------------------ bf16
DEV float bf16_to_f32(uint32_t u16) { return __uint_as_float(u16 << 16); }

// Two float32 -> packed bf16 (lo in bits 0..15), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
DEV uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

DEV uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// max(v, 0) with +0 for every v <= 0: as integers, the bit patterns of
// negative floats (and -0) are negative, so one integer max does it.
DEV float relu(float v) { return __int_as_float(max(__float_as_int(v), 0)); }

// ------------------------------------------------------------------ hashing
// SplitMix64 output finalizer (Steele, Lea, Flood 2014).
DEV uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

// ------------------------------------------------------- work-unit mapping
DEV uint64_t gcd_u64(uint64_t a, uint64_t b) {
  while (b) {
    uint64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// Test-only launch-order perturbation: a seeded affine bijection of [0, U)
// plus a seeded delay for some workgroups.
DEV int64_t shuffle_unit(int64_t L, int64_t U, uint64_t seed) {
  uint64_t h = mix64(seed);
  uint64_t a = (h % (uint64_t)U) | 1ull;
  while (gcd_u64(a, (uint64_t)U) != 1ull) a += 2;
  uint64_t c = mix64(h ^ kGamma) % (uint64_t)U;
  return (int64_t)((a * (uint64_t)L + c) % (uint64_t)U);
}

DEV void shuffle_delay(uint64_t seed, int64_t b) {
  uint64_t h = mix64(seed ^ ((uint64_t)b * kGamma));
  if ((h & 3u) == 0) {
    int n = (int)((h >> 8) & 15u);
    for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(32);
  }
}

// Maps the physical workgroup index b to a logical work unit in [0, U), or
// -1 when this workgroup has no unit.  Workgroups are dealt round-robin to
// the 8 XCDs, so unit ranges are laid out per XCD: XCD x takes the
// consecutive units [x*per, (x+1)*per), which keeps units that share
// operands in one L2.  With a nonzero seed the units are permuted instead.
DEV int64_t map_unit(int64_t b, int64_t U, uint64_t seed) {
  if (U <= 0) return -1;
  const int64_t per = (U + kNumXcd - 1) / kNumXcd;
  const int64_t x = b % kNumXcd, q = b / kNumXcd;
  if (q >= per) return -1;
  int64_t L = x * per + q;
  if (L >= U) return -1;
  if (seed) {
    shuffle_delay(seed, b);
    L = shuffle_unit(L, U, seed);
  }
  return L;
}

// Work-unit mapping for kernels whose units are ordered most expensive
// first and whose workgroups each fill a compute unit: the first round
// (units [0, min(U, ncu))) and the remaining units are each laid out per XCD
// as in map_unit, so the cheap units at the end of the order run last on
// every XCD.  The grid must hold round_up8(min(U, ncu)) + round_up8(U - ncu)
// workgroups (at most round_up8(U) + 8).
DEV int64_t map_unit_rounds(int64_t b, int64_t U, int ncu, uint64_t seed) {
  if (U <= 0) return -1;
  const int64_t U1 = U < ncu ? U : ncu;
  const int64_t per1 = (U1 + kNumXcd - 1) / kNumXcd;
  int64_t L;
  if (b < per1 * kNumXcd) {
    const int64_t q = b / kNumXcd;
    L = (b % kNumXcd) * per1 + q;
    if (L >= U1) return -1;
  } else {
    const int64_t b2 = b - per1 * kNumXcd, U2 = U - U1;
    const int64_t per2 = (U2 + kNumXcd - 1) / kNumXcd;
    const int64_t q = b2 / kNumXcd;
    if (q >= per2) return -1;
    L = U1 + (b2 % kNumXcd) * per2 + q;
    if (L >= U) return -1;
  }
  if (seed) {
    shuffle_delay(seed, b);
    L = shuffle_unit(L, U, seed);
  }
  return L;
}

// ------------------------------------------------------------ block scans
// Exclusive prefix over G values computed by val(g), written to s_pre[0..G]
// (s_pre[G] = total).  All NT threads of the block must call it; ends with a
// barrier.  Integer arithmetic: exact and order-independent.
template <int NT, class F, class T = int>
DEV void block_exclusive_scan(T* s_pre, T* s_tmp, int G, F val) {
  const int tid = threadIdx.x;
  const int per = (G + NT - 1) / NT;
  const int g0 = tid * per;
  T local = 0;
  for (int i = 0; i < per; ++i) {
    int g = g0 + i;
    if (g < G) local += (T)val(g);
  }
  // wave inclusive scan of per-thread sums
  const int lane = tid & (kWave - 1), w = tid / kWave;
  T incl = local;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    T o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) s_tmp[w] = incl;
  __syncthreads();
  T wbase = 0;
  for (int i = 0; i < w; ++i) wbase += s_tmp[i];
  T run = wbase + incl - local;
  for (int i = 0; i < per; ++i) {
    int g = g0 + i;
    if (g < G) {
      s_pre[g] = run;
      run += (T)val(g);
    }
  }
  if (tid == NT - 1) {
    T tot = 0;
    for (int i = 0; i < NT / kWave; ++i) tot += s_tmp[i];
    s_pre[G] = tot;
  }
  __syncthreads();
}

// Largest g in [0, G) with pre[g] <= L (pre non-decreasing, pre[0] = 0,
// L < pre[G]); skips empty groups.
DEV int find_group(const int* pre, int G, int64_t L) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= L)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// find_group over the values key(pre[g]).
template <class T, class Key>
DEV int find_group_by(const T* pre, int G, int64_t L, Key key) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (key(pre[mid]) <= L)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

}  // namespace moedet
