// fp32 grouped-GEMM building blocks for gfx950 (the float32-storage path).
//
// Tile 64x64x16, 4 waves in a 2x2 grid, each wave one
// v_mfma_f32_32x32x2f32 block.  Operands are staged global -> VGPR -> LDS
// with the tile stored [MN rows][K] (K contiguous, rows padded to 17 floats):
// K-contiguous sources are copied 4 floats at a time, M/N-contiguous sources
// are transposed on the way into LDS.
#pragma once

#include "common.h"

namespace moedet {
namespace f32 {

constexpr int BM = 64, BN = 64, BK = 16, NT = 256, ROW = 17;
constexpr int OPER = 64 * ROW;
constexpr int LDS_BYTES = 4 * OPER * 4;

DEV void zero_acc(f32x16_t& acc) {
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
}

// acc lane l holds C[m = l%32][n = 8*(r/4) + 4*(l/32) + r%4] of the wave's
// 32x32 block (B fragment passed as the MFMA's first operand).
DEV void mma_slice(const float* As, const float* Bs, f32x16_t& acc, int wm, int wn, int lane) {
  const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int k = kk * 2 + half;
    float a = As[(wm * 32 + r32) * ROW + k];
    float b = Bs[(wn * 32 + r32) * ROW + k];
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(b, a, acc, 0, 0, 0);
  }
}

// K-contiguous source: thread t copies 4 floats (k = 4*(t%4)..) of row t/4.
struct KcLoader {
  const float* rp;
  f32x4_t reg;
  DEV void init(int tid, const float* base, int64_t ld, const int32_t* rows, int64_t row0, int nvalid) {
    const int mn = tid >> 2;
    if (mn < nvalid) {
      const int64_t r = rows ? (int64_t)rows[row0 + mn] : row0 + mn;
      rp = base + r * ld + ((tid & 3) << 2);
    } else {
      rp = nullptr;
    }
  }
  DEV void load(int64_t k0) { reg = rp ? *(const f32x4_t*)(rp + k0) : f32x4_t{0.f, 0.f, 0.f, 0.f}; }
  DEV void store(float* s, int tid) const {
    const int mn = tid >> 2, k = (tid & 3) << 2;
#pragma unroll
    for (int q = 0; q < 4; ++q) s[mn * ROW + k + q] = reg[q];
  }
};

// M/N-contiguous source: thread t loads 4 mn values (mn = 4*(t%16)..) of K
// row t/16; rowptr(k) gives the row (pointer to element mn0) or nullptr.
struct MncLoader {
  f32x4_t reg;
  template <class RowPtr>
  DEV void load(int tid, RowPtr rowptr) {
    const int k = tid >> 4, mn = (tid & 15) << 2;
    const float* p = rowptr(k);
    reg = p ? *(const f32x4_t*)(p + mn) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  DEV void store(float* s, int tid) const {
    const int k = tid >> 4, mn = (tid & 15) << 2;
#pragma unroll
    for (int q = 0; q < 4; ++q) s[(mn + q) * ROW + k] = reg[q];
  }
};

}  // namespace f32
}  // namespace moedet
