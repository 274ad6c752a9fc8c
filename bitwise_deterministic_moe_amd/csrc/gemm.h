// Grouped-GEMM building blocks for gfx950: tile configurations, global->LDS
// loaders and the MFMA main loop shared by the expert GEMM kernels.
//
// Every operand tile lives in LDS as [MN rows][BK] with K contiguous, which
// is the order an MFMA lane consumes it in (8 consecutive k per lane for
// bf16, 1 for fp32).  Sources that are contiguous along K are copied
// 16 bytes at a time; sources contiguous along M/N are transposed in
// registers (8x8 blocks of 16-bit values) on their way into LDS.
#pragma once

#include "common.h"

namespace moedet {

template <typename T>
struct Tile;

// bf16: 256x256x64 tiles, 4 waves in a 2x2 grid, each wave 128x128 made of
// 4x4 blocks of v_mfma_f32_32x32x16_bf16.  LDS rows are 128 bytes without
// padding; the 16-byte chunk c of row r is stored at chunk c ^ swz(r), which
// keeps both the 16-byte stores and the MFMA fragment reads free of bank
// conflicts for 32- and 64-bank LDS.
template <>
struct Tile<uint16_t> {
  static constexpr int BM = 256, BN = 256, BK = 64, NT = 256;
  static constexpr int WM = 2, WN = 2, MB = 4, NB = 4;
  static constexpr int KSTEP = 16;                  // MFMA K
  static constexpr int OPER_ELEMS = 256 * 64;       // one operand stage
  static constexpr int LDS_BYTES = 4 * OPER_ELEMS * 2;
};

// fp32: 64x64x16 tiles, 4 waves in a 2x2 grid, each wave one
// v_mfma_f32_32x32x2f32 block.  LDS rows padded to 17 floats.
template <>
struct Tile<float> {
  static constexpr int BM = 64, BN = 64, BK = 16, NT = 256;
  static constexpr int WM = 2, WN = 2, MB = 1, NB = 1;
  static constexpr int KSTEP = 2;
  static constexpr int ROW = 17;
  static constexpr int OPER_ELEMS = 64 * 17;
  static constexpr int LDS_BYTES = 4 * OPER_ELEMS * 4;
};

DEV int swz(int r) { return (r + (r >> 3)) & 7; }

// Offset (in elements) of the 16-byte chunk c of LDS row r (bf16 tiles).
DEV int lds_chunk_off(int r, int c) { return r * 64 + ((c ^ swz(r)) << 3); }

DEV u32x4_t zero4() { return u32x4_t{0u, 0u, 0u, 0u}; }

// relu(v)^2 on the 8 bf16 values of a 16-byte chunk, rounded back to bf16.
DEV u32x4_t act_bf16x8(u32x4_t v) {
  u32x4_t o;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float lo = relu(bf16_to_f32(v[w] & 0xffffu));
    float hi = relu(bf16_to_f32(v[w] >> 16));
    o[w] = pack_bf16x2(lo * lo, hi * hi);
  }
  return o;
}

DEV u32x4_t scale_bf16x8(u32x4_t v, float s) {
  u32x4_t o;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    o[w] = pack_bf16x2(bf16_to_f32(v[w] & 0xffffu) * s, bf16_to_f32(v[w] >> 16) * s);
  return o;
}

// 8x8 transpose of 16-bit values: in[j] holds row j (8 values, 2 per
// word), out[i] receives column i.
DEV void transpose8x8(const u32x4_t in[8], u32x4_t out[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int wsel = i >> 1;
    const bool hi = i & 1;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t a = in[2 * w][wsel], b = in[2 * w + 1][wsel];
      out[i][w] = hi ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
  }
}

// ------------------------------------------------------------ MFMA tile
// Accumulates one BK slice held in LDS into the wave's accumulators.
// acc[mb][nb] lane l holds C[m = mb*32 + l%32][n = nb*32 + 8*(r/4) + 4*(l/32) + r%4]
// (relative to the wave's corner): the B fragment is passed as the MFMA's
// first operand so that each lane ends with runs of 4 consecutive columns.
template <typename T>
DEV void mma_slice(const T* As, const T* Bs, f32x16_t (&acc)[Tile<T>::MB][Tile<T>::NB], int wm,
                   int wn, int lane);

template <>
DEV void mma_slice<uint16_t>(const uint16_t* As, const uint16_t* Bs, f32x16_t (&acc)[4][4], int wm,
                             int wn, int lane) {
  const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    bf16x8_t af[4], bf[4];
    const int c = kk * 2 + half;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int r = wm * 128 + mb * 32 + r32;
      af[mb] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(As + lds_chunk_off(r, c)));
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int r = wn * 128 + nb * 32 + r32;
      bf[nb] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(Bs + lds_chunk_off(r, c)));
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[nb], af[mb], acc[mb][nb], 0, 0, 0);
  }
}

template <>
DEV void mma_slice<float>(const float* As, const float* Bs, f32x16_t (&acc)[1][1], int wm, int wn,
                          int lane) {
  const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int k = kk * 2 + half;
    float a = As[(wm * 32 + r32) * 17 + k];
    float b = Bs[(wn * 32 + r32) * 17 + k];
    acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(b, a, acc[0][0], 0, 0, 0);
  }
}

// ------------------------------------------------------------ loaders
// K-contiguous source: tile row mn reads row_ptr(mn)[k0 .. k0+BK).
// bf16: thread t copies chunk t%8 of rows t/8 + 32*i (i = 0..7).
// fp32: thread t copies 4 floats (k = 4*(t%4)..) of row t/4.
template <typename T, bool ACT>
struct KcLoader;

template <bool ACT>
struct KcLoader<uint16_t, ACT> {
  const uint16_t* rp[8];  // row pointers (nullptr: row outside the group -> zeros)
  u32x4_t reg[8];
  DEV void init(int tid, const uint16_t* base, int64_t ld, const int32_t* rows, int64_t row0,
                int nvalid, bool gather) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int mn = (tid >> 3) + 32 * i;
      if (mn < nvalid) {
        int64_t r = gather ? (int64_t)rows[row0 + mn] : row0 + mn;
        rp[i] = base + r * ld + ((tid & 7) << 3);
      } else {
        rp[i] = nullptr;
      }
    }
  }
  DEV void load(int64_t k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) reg[i] = rp[i] ? *(const u32x4_t*)(rp[i] + k0) : zero4();
  }
  DEV void store(uint16_t* s, int tid) const {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int mn = (tid >> 3) + 32 * i;
      *(u32x4_t*)(s + lds_chunk_off(mn, tid & 7)) = ACT ? act_bf16x8(reg[i]) : reg[i];
    }
  }
};

template <bool ACT>
struct KcLoader<float, ACT> {
  const float* rp;
  f32x4_t reg;
  DEV void init(int tid, const float* base, int64_t ld, const int32_t* rows, int64_t row0,
                int nvalid, bool gather) {
    const int mn = tid >> 2;
    if (mn < nvalid) {
      int64_t r = gather ? (int64_t)rows[row0 + mn] : row0 + mn;
      rp = base + r * ld + ((tid & 3) << 2);
    } else {
      rp = nullptr;
    }
  }
  DEV void load(int64_t k0) { reg = rp ? *(const f32x4_t*)(rp + k0) : f32x4_t{0.f, 0.f, 0.f, 0.f}; }
  DEV void store(float* s, int tid) const {
    const int mn = tid >> 2, k = (tid & 3) << 2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v = reg[q];
      if (ACT) {
        v = relu(v);
        v = v * v;
      }
      s[mn * 17 + k + q] = v;
    }
  }
};

// MN-contiguous source: K row k (0 <= k < BK of the current slice) reads
// krow_ptr(k)[mn0 .. mn0+BM).  The caller supplies per-k row pointers via
// a functor; rows beyond the valid K range read as zeros.  Optional
// per-row scale (applied in fp32, rounded to bf16) or relu^2.
// bf16: thread t loads the 8x8 block (mn = 8*(t/8).., k = 8*(t%8)..).
// fp32: thread t loads 4 mn values (mn = 4*(t%16)..) of k row t/16.
template <typename T, bool ACT, bool SCALE>
struct MncLoader;

template <bool ACT, bool SCALE>
struct MncLoader<uint16_t, ACT, SCALE> {
  u32x4_t reg[8];
  // rowptr(k) -> pointer to element mn0 of K row k, or nullptr; scale(k).
  template <class RowPtr, class Scale>
  DEV void load(int tid, RowPtr rowptr, Scale scale) {
    const int c = tid & 7, G = tid >> 3;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint16_t* p = rowptr(8 * c + j);
      u32x4_t v = p ? *(const u32x4_t*)(p + 8 * G) : zero4();
      if (SCALE) v = p ? scale_bf16x8(v, scale(8 * c + j)) : v;
      if (ACT) v = act_bf16x8(v);
      reg[j] = v;
    }
  }
  DEV void store(uint16_t* s, int tid) const {
    const int c = tid & 7, G = tid >> 3;
    u32x4_t t[8];
    transpose8x8(reg, t);
#pragma unroll
    for (int i = 0; i < 8; ++i) *(u32x4_t*)(s + lds_chunk_off(8 * G + i, c)) = t[i];
  }
};

template <bool ACT, bool SCALE>
struct MncLoader<float, ACT, SCALE> {
  f32x4_t reg;
  template <class RowPtr, class Scale>
  DEV void load(int tid, RowPtr rowptr, Scale scale) {
    const int k = tid >> 4, mn = (tid & 15) << 2;
    const float* p = rowptr(k);
    f32x4_t v = p ? *(const f32x4_t*)(p + mn) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (SCALE && p) {
      const float s = scale(k);
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] *= s;
    }
    if (ACT) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float r = relu(v[q]);
        v[q] = r * r;
      }
    }
    reg = v;
  }
  DEV void store(float* s, int tid) const {
    const int k = tid >> 4, mn = (tid & 15) << 2;
#pragma unroll
    for (int q = 0; q < 4; ++q) s[(mn + q) * 17 + k] = reg[q];
  }
};

template <typename T>
DEV void zero_acc(f32x16_t (&acc)[Tile<T>::MB][Tile<T>::NB]) {
#pragma unroll
  for (int a = 0; a < Tile<T>::MB; ++a)
#pragma unroll
    for (int b = 0; b < Tile<T>::NB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
}

}  // namespace moedet
