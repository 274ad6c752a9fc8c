// Expert grouped GEMMs for gfx950.
//
//  rowgemm  C[rows of expert g, N] = A[rows, K] * B_g, K = D or F:
//           fc1 forward   A = x[row_tok] (K-contig), B = W1_g [D][F] (N-contig),
//                         epilogue stores h and a = relu(h)^2;
//           fc2 forward   A = a, B = W2_g [F][D];
//           fc2 dgrad     A = dy[row_tok], B = W2_g read as [N=F][K=D],
//                         epilogue: dprob partial and dh;
//           fc1 dgrad     A = dh, B = W1_g read as [N=D][K=F].
//  wgrad    dW_g[M, N] = sum over the expert's rows of A_row^T B_row (both
//           operands contiguous along M/N), rows split into chunks whose size
//           depends on shapes only:
//           dW1 = x[row_tok]^T dh,   dW2 = act_p^T dy[row_tok], where
//           act_p = p relu(h)^2 is rebuilt from h by the weight-gradient
//           prologue kernel.
//
// Expert row counts live on the device: the permute scan turns them into
// the routing work list (row tiles longest first, weight-gradient units),
// which the workgroups of the bf16 kernels read (no host synchronisation);
// the grid is an upper bound and surplus workgroups exit at once.  The
// float32 weight-gradient kernels derive their units from counts[].
//
// Deterministic reductions (the English digest "Trillion-Parameter
// Pretraining Goes Bitwise-Deterministic", section "Interpretation"):
//  * dprob: each (row, N-tile) pair writes its own float32 partial; a
//    later pass adds the partials in N-tile order.  The atomic mode adds
//    them into dprob[token] directly, in arrival order.
//  * wgrad split-K: chunk partials go to the output (chunk 0) and to
//    workspace slots (chunks 1..S-1) and a later pass adds them in chunk
//    order; the atomic mode adds all chunks atomically into a zeroed dW.
#include <type_traits>

#include "gemm_bf16.h"
#include "gemm_f32.h"
#include "kernels.h"

namespace moedet {

// ------------------------------------------------------------ element I/O
template <typename T>
DEV float round_t(float v);
template <>
DEV float round_t<uint16_t>(float v) { return bf16_to_f32(f32_to_bf16(v)); }
template <>
DEV float round_t<float>(float v) { return v; }

DEV void load4(const uint16_t* p, float (&v)[4]) {
  u32x2_t x = *(const u32x2_t*)p;
  v[0] = bf16_to_f32(x[0] & 0xffffu);
  v[1] = bf16_to_f32(x[0] >> 16);
  v[2] = bf16_to_f32(x[1] & 0xffffu);
  v[3] = bf16_to_f32(x[1] >> 16);
}
DEV void load4(const float* p, float (&v)[4]) {
  f32x4_t x = *(const f32x4_t*)p;
  v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
}
DEV void store4(uint16_t* p, const float (&v)[4]) {
  *(u32x2_t*)p = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
DEV void store4(float* p, const float (&v)[4]) { *(f32x4_t*)p = f32x4_t{v[0], v[1], v[2], v[3]}; }

// Buffer resource covering [p, p + 2^31); offsets >= 2^31 are dropped on
// store and read as zero on load.  Arrays indexed by routed row can exceed
// 2 GiB, so their resources start at the first row a tile touches
// (tile_rows), and offsets within a tile stay far below 2^31.
DEV __amdgpu_buffer_rsrc_t buf(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, 0x7fffffff, 0x00020000);
}
// Row `row` of a row-major array of `ld` elements of `es` bytes per row.
DEV const void* row_ptr(const void* p, int64_t row, int64_t ld, int es) {
  return (const char*)p + row * ld * es;
}
DEV __amdgpu_buffer_rsrc_t tile_rows(const void* p, int64_t row0, int64_t ld, int es) {
  return buf(row_ptr(p, row0, ld, es));
}
constexpr uint32_t kNoRow = 0x80000000u;
// Cache policy of the epilogue's loads and stores: non-temporal.  Each
// output element is written once and each h element read once per launch;
// streaming them keeps the L2 for the operand tiles that several workgroups
// of an XCD share (measured: fc2 dgrad 85 -> 78 us on the bf16 8x2 workload).
constexpr int kEpiNT = 2;

// Sum over the 4 lanes of each quad with two DPP butterflies (lane pairs
// (0,1)(2,3), then (0,2)(1,3)); a + b == b + a, so all four lanes end with
// the same bits.
DEV float quad_sum(float v) {
  v = v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v = v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  return v;
}

// ------------------------------------------------------------ row tiles
struct RowTile {
  int g, m0, n0, nt, mvalid;
  int64_t off;
};

// Work unit of this workgroup: (row tile, n-tile), a side unit, or nothing.
// Row tiles come from the routing work list (longest first: full tiles, then
// partial tiles by descending rows), so when units outnumber compute units
// the last, short round holds the smallest tiles.
enum { kTileNone = 0, kTileGemm = 1, kTileSide = 2 };
template <int BMv, int BNv>
DEV int row_tile(const RowGemmParams& P, RowTile& t) {
  if (P.side_units > 0 && (int64_t)blockIdx.x >= P.gemm_grid) {
    t.nt = (int)(blockIdx.x - P.gemm_grid);  // side unit index
    return t.nt < P.side_units ? kTileSide : kTileNone;
  }
  const int nN = P.N / BNv;
  const int64_t U = (int64_t)P.sched[P.list_hdr] * nN;
  const int64_t L = map_unit_rounds(blockIdx.x, U, P.ncu, P.seed);
  if (L < 0) return kTileNone;
  // L < 2^31 (one unit per workgroup of the grid): 32-bit division
  const int64_t mt = (uint32_t)L / (uint32_t)nN;
  t.nt = (int)((uint32_t)L % (uint32_t)nN);
  const int4 en = ((const int4*)(P.sched + P.list_at))[mt];
  t.g = __builtin_amdgcn_readfirstlane(en.x);
  t.m0 = __builtin_amdgcn_readfirstlane(en.y);
  t.off = (int64_t)__builtin_amdgcn_readfirstlane(en.z - en.y);
  t.mvalid = __builtin_amdgcn_readfirstlane(en.w);
  t.nt = __builtin_amdgcn_readfirstlane(t.nt);
  t.n0 = t.nt * BNv;
  return kTileGemm;
}

// Side unit u: the dprob combine of flat slots [u*kSideSlots, ...), one
// thread per slot.  The n_tiles partials of the slot's row are added as a
// fixed pairwise tree over GS = next_pow2(n_tiles) positions (missing ones
// are 0): level d adds position q + d into q for q = 0, 2d, 4d, ...  The
// tree depends on n_tiles only.  Slots of non-local experts get 0.
template <int GS>
DEV float tree_sum(const float* pr, int n) {
  float v[GS];
#pragma unroll
  for (int q = 0; q < GS; ++q) v[q] = q < n ? pr[q] : 0.f;
#pragma unroll
  for (int d = 1; d < GS; d <<= 1)
#pragma unroll
    for (int q = 0; q < GS; q += 2 * d) v[q] = v[q] + v[q + d];
  return v[0];
}

DEV void dprob_side(const RowGemmParams& P, int u) {
  int gs = 1;
  while (gs < P.n_tiles) gs <<= 1;
  const int64_t s0 = (int64_t)u * kSideSlots;
#pragma unroll 4
  for (int j = threadIdx.x; j < kSideSlots; j += 256) {
    const int64_t i = s0 + j;
    if (i >= P.side_nslot) break;
    const int32_t r = P.side_slot_row[i];
    float out = 0.f;
    if (r >= 0) {
      const float* pr = P.part + (int64_t)r * P.n_tiles;
      switch (gs) {
        case 1: out = tree_sum<1>(pr, P.n_tiles); break;
        case 2: out = tree_sum<2>(pr, P.n_tiles); break;
        case 4: out = tree_sum<4>(pr, P.n_tiles); break;
        case 8: out = tree_sum<8>(pr, P.n_tiles); break;
        case 16: out = tree_sum<16>(pr, P.n_tiles); break;
        case 32: out = tree_sum<32>(pr, P.n_tiles); break;
        default: out = tree_sum<64>(pr, P.n_tiles); break;
      }
    }
    P.dprob[i] = out;
  }
}

// Epilogue over the accumulators (layout documented in gemm_bf16.h /
// gemm_f32.h): acc[mb][nb] lane l holds row wm*WTM + mb*32 + l%32 and columns
// wn*WTN + nb*32 + 8*i + 4*(l/32) + 0..3 in registers 4i..4i+3.
template <typename T, int MB, int NB, int WTM, int WTN, int BMv, int WN, int EPI>
DEV void row_epilogue(const RowGemmParams& P, const RowTile& t, f32x16_t (&acc)[MB][NB], float* s_part, int wm,
                      int wn, int lane, int tid) {
  const int r32 = lane & 31, half = lane >> 5;
  if constexpr (EPI == kEpiStore || EPI == kEpiStoreAct) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = wm * WTM + mb * 32 + r32;
      if (m >= t.mvalid) continue;
      const int64_t grow = t.off + t.m0 + m;
      T* crow = (T*)P.c + grow * P.ldc + t.n0 + wn * WTN;
      T* arow = (T*)P.c2 + grow * P.ldc2 + t.n0 + wn * WTN;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = nb * 32 + 8 * i + 4 * half;
          float v[4] = {acc[mb][nb][4 * i], acc[mb][nb][4 * i + 1], acc[mb][nb][4 * i + 2], acc[mb][nb][4 * i + 3]};
          store4(crow + n, v);
          if constexpr (EPI == kEpiStoreAct) {
            // activation of the stored (rounded) h, the value the backward sees
            float a[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float r = relu(round_t<T>(v[q]));
              a[q] = r * r;
            }
            store4(arow + n, a);
          }
        }
    }
  } else {
    // fc2 dgrad: acc = G = dy W2^T for rows m, columns f of this N-tile.
    //   part[row][nt] = sum_f G * relu(h)^2   (fixed order: nb, i, q inside a
    //                   lane; then the lane pair; then waves wn = 0, 1, ...)
    //   dh = (2 p G) * relu(h)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = wm * WTM + mb * 32 + r32;
      float part = 0.f;
      if (m < t.mvalid) {
        const int64_t grow = t.off + t.m0 + m;
        const float p = P.row_prob[grow];
        const float p2 = 2.f * p;
        const int64_t col = t.n0 + wn * WTN;
        const T* hrow = (const T*)P.h + grow * P.ldh + col;
        T* drow = (T*)P.c + grow * P.ldc + col;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = nb * 32 + 8 * i + 4 * half;
            float hv[4], dh[4];
            load4(hrow + n, hv);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float gq = acc[mb][nb][4 * i + q];
              const float rh = relu(hv[q]);
              part = __builtin_fmaf(gq, rh * rh, part);
              dh[q] = (p2 * gq) * rh;
            }
            store4(drow + n, dh);
          }
      }
      // lanes l and l^32 hold the two column halves of the same row;
      // a + b == b + a, so both get the same bits.
      part = part + __shfl_xor(part, 32, 64);
      if (half == 0) s_part[wn * BMv + m] = part;
    }
    __syncthreads();
    for (int m = tid; m < t.mvalid; m += 256) {
      float v = s_part[m];
#pragma unroll
      for (int w = 1; w < WN; ++w) v = v + s_part[w * BMv + m];
      const int64_t grow = t.off + t.m0 + m;
      if (P.atomic)
        atomicAdd(P.dprob + P.row_src[grow], v);
      else
        P.part[grow * P.n_tiles + t.nt] = v;
    }
  }
}

// Stores of a wgrad tile: direct, into a workspace slot, or atomic adds.
template <int MB, int NB, int WTM, int WTN>
DEV void wgrad_store(float* dst, int ldd, bool atomic_add, int m0, int n0, f32x16_t (&acc)[MB][NB], int wm, int wn,
                     int lane) {
  const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = m0 + wm * WTM + mb * 32 + r32;
    float* crow = dst + (int64_t)m * ldd + n0 + wn * WTN;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = nb * 32 + 8 * i + 4 * half;
        const f32x16_t& a = acc[mb][nb];
        if (atomic_add) {
#pragma unroll
          for (int q = 0; q < 4; ++q) atomicAdd(crow + n + q, a[4 * i + q]);
        } else {
          *(f32x4_t*)(crow + n) = f32x4_t{a[4 * i], a[4 * i + 1], a[4 * i + 2], a[4 * i + 3]};
        }
      }
  }
}

struct WgradTile {
  int g, s, S, klen, m0, n0;
  int64_t row0;
};

template <int BMv, int BNv>
DEV bool wgrad_tile(const WgradParams& P, WgradTile& t) {
  const int G = P.groups;
  const int nN = P.N / BNv;
  const int tiles = (P.M / BMv) * nN;
  const int32_t* unit_start = P.sched;
  const int64_t U = (int64_t)unit_start[G] * tiles;
  const int64_t L = map_unit(blockIdx.x, U, P.seed);
  if (L < 0) return false;
  const int64_t u = (uint32_t)L / (uint32_t)tiles;  // L < 2^31
  const int tile = (int)((uint32_t)L % (uint32_t)tiles);
  t.g = find_group(unit_start, G, u);
  t.s = (int)(u - unit_start[t.g]);
  const int cnt = P.counts[t.g];
  t.S = cnt > P.kc ? (cnt + P.kc - 1) / P.kc : 1;
  const int k_lo = (int)((int64_t)t.s * cnt / t.S), k_hi = (int)((int64_t)(t.s + 1) * cnt / t.S);
  t.klen = k_hi - k_lo;
  t.row0 = (int64_t)P.offsets[t.g] + k_lo;
  t.m0 = (tile / nN) * BMv;
  t.n0 = (tile % nN) * BNv;
  return true;
}

DEV float* wgrad_dst(const WgradParams& P, const WgradTile& t) {
  const int32_t* slot_base = P.sched + (P.groups + 1);
  if (!P.atomic && t.s > 0) return P.slots + (int64_t)(slot_base[t.g] + t.s - 1) * P.M * P.N;
  return P.dw + (int64_t)t.g * P.M * P.N;
}

// ================================================================= bf16
// Epilogues of the bf16 kernels go through LDS so that every global load and
// store is row-contiguous: the 256x256 float32 accumulator tile is written to
// LDS in four passes of 64 rows (row stride 260 floats); after each pass all
// 256 threads walk the 64 rows, four rows per step, each thread owning four
// consecutive columns (a wave covers one full row).
constexpr int kStageRow = 260;                       // floats per staged row
constexpr int kStageBytes = 64 * kStageRow * 4;      // 66,560 bytes, inside the main-loop ring
static_assert(kStageBytes <= bf::LDS_BYTES, "epilogue stage must fit in the ring");

// Pass p covers tile rows 64p..64p+63.  In step st (0..15) of a pass,
// thread tid owns row 64p + 4*st + tid/64 and columns 4*(tid%64)..+3, so
// each wave handles one whole row per step and control flow is uniform per
// wave.  Between passes only LDS traffic has to be ordered, so the barriers
// wait on LDS operations alone and global stores stay in flight.
// Everything is fully unrolled so that per-step data lives in registers.
DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
DEV int staged_row(int p, int st, int tid) {
  return 64 * p + 4 * st + __builtin_amdgcn_readfirstlane(tid >> 6);  // one row per wave
}
DEV int staged_col(int tid) { return (tid & 63) * 4; }

// pre.load(d, p): issue this thread's global loads needed by pass p into d
// (called one pass ahead; pass 0's by the caller when first_loaded);
// emit(row, col, v, d, st): consume one step.  Passes whose 64
// rows are all past `rows` (the tile's valid rows) are skipped (the decision
// is uniform over the workgroup).
// WTM: rows of a wave's tile (128, or 96 for a 192-row tile); a wave's
// 32-row block mb (tile rows wm*WTM + 32 mb ..) goes to the pass holding it.
template <int WTM = 128, class Pre, class Emit>
DEV void staged_epilogue(float* stage, f32x16_t (&acc)[4][4], int wm, int wn, int lane, int tid, int rows, Pre& pre,
                         typename Pre::Data (&d)[2], bool first_loaded, Emit emit) {
  const int r32 = lane & 31, half = lane >> 5;
  const int npass = rows >= 2 * WTM ? 2 * WTM / 64 : (rows + 63) / 64;
  if (npass > 0 && !first_loaded) pre.load(d[0], 0);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if (p < npass) {
#pragma unroll
      for (int mb = 0; mb < WTM / 32; ++mb) {
        const int r0 = wm * WTM + mb * 32 - 64 * p;  // block start within the pass (uniform)
        if (r0 >= 0 && r0 < 64) {
          const int m = r0 + r32;  // row within the pass
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int n = wn * 128 + nb * 32 + 8 * i + 4 * half;
              const f32x16_t& a = acc[mb][nb];
              *(f32x4_t*)(stage + m * kStageRow + n) = f32x4_t{a[4 * i], a[4 * i + 1], a[4 * i + 2], a[4 * i + 3]};
            }
        }
      }
      lds_barrier();
      if (p + 1 < npass) pre.load(d[(p + 1) & 1], p + 1);
      f32x4_t v[16];
#pragma unroll
      for (int st = 0; st < 16; ++st)
        v[st] = *(const f32x4_t*)(stage + (4 * st + (tid >> 6)) * kStageRow + staged_col(tid));
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        float f[4] = {v[st][0], v[st][1], v[st][2], v[st][3]};
        emit(staged_row(p, st, tid), staged_col(tid), f, d[p & 1], st);
      }
      lds_barrier();
    }
  }
}

struct NoPre {
  struct Data {};
  DEV void load(Data&, int) {}
};

// Main loop instantiated for the number of the wave's A blocks that hold
// rows, so that the waves of a partial tile skip MFMAs on zero rows while
// every variant stays straight-line code.
template <int AL, int BL, int NS, int WTM, class Issue>
DEV void run_mainloop(int nmb, const uint16_t* lds, uint32_t ring, int nsteps, Issue issue, f32x16_t (&acc)[4][4],
                      int wm, int wn, int lane) {
  switch (nmb) {
    case 0: bf::mainloop<AL, BL, 0, NS, WTM>(lds, ring, nsteps, issue, acc, wm, wn, lane); break;
    case 1: bf::mainloop<AL, BL, 1, NS, WTM>(lds, ring, nsteps, issue, acc, wm, wn, lane); break;
    case 2: bf::mainloop<AL, BL, 2, NS, WTM>(lds, ring, nsteps, issue, acc, wm, wn, lane); break;
    case 3: bf::mainloop<AL, BL, 3, NS, WTM>(lds, ring, nsteps, issue, acc, wm, wn, lane); break;
    default:
      if constexpr (WTM >= 128) bf::mainloop<AL, BL, 4, NS, WTM>(lds, ring, nsteps, issue, acc, wm, wn, lane);
      break;
  }
}

// Ring depth per tile (uniform over the workgroup): a tile with at most 128
// rows has too few MFMAs per slice to cover the load latency with 4 slots
// and takes 5; fuller tiles keep 4 (measured: the deeper ring slows them).
template <int AL, int BL, int WTM, class Issue>
DEV void run_row_mainloop(int mvalid, int nmb, const uint16_t* lds, uint32_t ring, int nsteps, Issue issue,
                          f32x16_t (&acc)[4][4], int wm, int wn, int lane) {
  if (mvalid <= 128)
    run_mainloop<AL, BL, 5, WTM>(nmb, lds, ring, nsteps, issue, acc, wm, wn, lane);
  else
    run_mainloop<AL, BL, 4, WTM>(nmb, lds, ring, nsteps, issue, acc, wm, wn, lane);
}

// Loads of h for the fc2 dgrad epilogue: pass p, step st reads the 4
// columns of this thread in tile row staged_row(p, st) (rows past the tile's
// valid rows read zeros).
struct HPre {
  struct Data {
    u32x2_t h[16];
  };
  const RowGemmParams& P;
  const RowTile& t;
  int tid;
  DEV void load(Data& d, int p) {
    const __amdgpu_buffer_rsrc_t rh = tile_rows(P.h, t.off + t.m0, P.ldh, 2);
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int m = staged_row(p, st, tid);
      const bool ok = m < t.mvalid;
      d.h[st] = __builtin_amdgcn_raw_buffer_load_b64(
          rh, ok ? ((uint32_t)m * (uint32_t)P.ldh + t.n0 + staged_col(tid)) * 2u : kNoRow, 0, kEpiNT);
    }
  }
};

// Row GEMMs hold a 5-slot ring (all 160 KiB of LDS); after the main loop
// the ring holds the epilogue stage, then the quad sums and row
// probabilities of the fc2 dgrad epilogue.
constexpr int kRowNS = 5;
constexpr int kQsumOff = kStageBytes;                     // float [BM][16]
constexpr int kProbOff = kQsumOff + bf::BM * 16 * 4;      // float [BM]
static_assert(kProbOff + bf::BM * 4 <= bf::ring_bytes<kRowNS>, "epilogue scratch must fit in the ring");

// fc2 dgrad epilogue (shared by the bf16 and the MXFP8 row GEMMs):
// v = G = dy W2^T at (row, columns col..col+3 of this N-tile).
//   part[row][nt] = sum over the tile's 256 columns of G * relu(h)^2:
//                   4 columns in order inside a lane, a DPP butterfly over
//                   the lane quad (16 columns), then the 16 quad sums of
//                   the row in quad order (through LDS);
//   dh = (2 p G) * relu(h).
// h of a pass is loaded one pass ahead; the row probabilities come from
// LDS.  lds: the main-loop ring, free (the main loop ended with a barrier).
template <int WTM>
DEV void dgrad2_epilogue(const RowGemmParams& P, const RowTile& t, uint16_t* lds, f32x16_t (&acc)[4][4], int wm,
                         int wn, int lane, int tid, float my_prob) {
  float* stage = (float*)lds;
  float* s_qsum = (float*)((char*)lds + kQsumOff);  // [tile row][quad]
  float* s_prob = (float*)((char*)lds + kProbOff);
  s_prob[tid] = my_prob;  // the main loop ended with a barrier: the ring is free
  lds_barrier();
  HPre hpre{P, t, tid};
  HPre::Data hd[2];
  const __amdgpu_buffer_rsrc_t rc = tile_rows(P.c, t.off + t.m0, P.ldc, 2);
  staged_epilogue<WTM>(stage, acc, wm, wn, lane, tid, t.mvalid, hpre, hd, false, [&](int m, int col, float (&g)[4], HPre::Data& d, int st) {
    const bool valid = m < t.mvalid;   // uniform across the wave (one row per wave)
    if (!valid) return;
    const float p2 = 2.f * s_prob[m];
    float hv[4], dh[4];
    hv[0] = bf16_to_f32(d.h[st][0] & 0xffffu);
    hv[1] = bf16_to_f32(d.h[st][0] >> 16);
    hv[2] = bf16_to_f32(d.h[st][1] & 0xffffu);
    hv[3] = bf16_to_f32(d.h[st][1] >> 16);
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float rh = relu(hv[q]);
      part = __builtin_fmaf(g[q], rh * rh, part);
      dh[q] = (p2 * g[q]) * rh;
    }
    const uint32_t o = (uint32_t)m * 2u * (uint32_t)P.ldc + (t.n0 + col) * 2u;
    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(dh[0], dh[1]), pack_bf16x2(dh[2], dh[3])}, rc, o, 0, kEpiNT);
    part = quad_sum(part);
    if ((lane & 3) == 0) s_qsum[m * 16 + (lane >> 2)] = part;
  });
  __syncthreads();
  // one thread per tile row: the 16 quad sums in order
  if (tid < t.mvalid) {
    float v = s_qsum[tid * 16];
#pragma unroll
    for (int q = 1; q < 16; ++q) v = v + s_qsum[tid * 16 + q];
    const int64_t grow = t.off + t.m0 + tid;
    if (P.atomic)
      atomicAdd(P.dprob + P.row_src[grow], v);
    else
      P.part[grow * P.n_tiles + t.nt] = v;
  }
}

// One row tile of the bf16 row GEMM, with WTM rows per wave row (128, or 96
// for a tile of at most 192 rows: then both wave rows hold three 32-row
// blocks instead of four and at most two, so the slower wave does three
// quarters of the MFMAs).  The tile's LDS A operand always has 256 rows.
template <int BL, int EPI, int WTM>
DEV void rowgemm_bf16_tile(const RowGemmParams& P, const RowTile& t, uint16_t* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t ring = bf::lds_base(lds);
  const int wm = wave >> 1, wn = wave & 1;
  // routing probability of each tile row (fc2 dgrad epilogue); loaded now,
  // stored to LDS once the ring is free
  float my_prob = 0.f;
  if constexpr (EPI == kEpiDgrad2) my_prob = tid < t.mvalid ? P.row_prob[t.off + t.m0 + tid] : 0.f;

  bf::KcOperand oa;
  // A gathered by token: rows of a[T][lda] (below 2 GiB); else the tile's own
  // rows, addressed from the first.  Branch-free so that the four row-index
  // loads of a thread are in flight together (the tile holds at least one
  // valid row).
  const bool gathered = P.a_rows != nullptr;
  const int64_t row0 = t.off + t.m0;
  oa.init(gathered ? P.a : row_ptr(P.a, row0, P.lda, 2),
          gathered ? P.a_bytes : (uint32_t)(t.mvalid * P.lda * 2), wave, lane, [&](int r) -> uint32_t {
    const int rc = r < t.mvalid ? r : t.mvalid - 1;
    const int64_t row = gathered ? (int64_t)P.a_rows[row0 + rc] : rc;
    return r < t.mvalid ? (uint32_t)(row * P.lda * 2) : bf::kOOB;
  });
  const uint16_t* Bg = (const uint16_t*)P.b + (int64_t)t.g * P.b_gstride;
  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  const int nsteps = P.K / bf::BK;
  // K is a positive multiple of 256 (checked at the boundary), so the main
  // loop's first MFMAs always run and the zeros above stay only in blocks of
  // rows past the tile's end
  __builtin_assume(nsteps > 0);
  // 32-row A blocks of this wave that hold rows (wave-uniform)
  const int nmb = max(0, min(WTM / 32, (t.mvalid - wm * WTM + 31) / 32));
  if constexpr (BL == bf::KC) {
    bf::KcOperand ob;
    ob.init(Bg, P.b_bytes, wave, lane, [&](int r) -> uint32_t { return (uint32_t)((t.n0 + r) * P.ldb * 2); });
    auto issue = [&](int s, uint32_t st, int i) {
      if (i < bf::LOADS)
        oa.issue1(st, wave, s * bf::BK, s < nsteps, i);
      else
        ob.issue1(st + bf::OPER * 2, wave, s * bf::BK, s < nsteps, i - bf::LOADS);
    };
    run_row_mainloop<bf::KC, bf::KC, WTM>(t.mvalid, nmb, lds, ring, nsteps, issue, acc, wm, wn, lane);
  } else {
    bf::MncOperand ob;
    ob.init(Bg, P.b_bytes, wave, lane, t.n0);
    // byte offset of this lane's k row of load j in slice 0
    uint32_t kro[bf::LOADS];
#pragma unroll
    for (int j = 0; j < bf::LOADS; ++j) kro[j] = (uint32_t)(bf::MncOperand::krow(wave, lane, j) * P.ldb * 2);
    const uint32_t slice_bytes = (uint32_t)(bf::BK * P.ldb * 2);
    auto issue = [&](int s, uint32_t st, int i) {
      if (i < bf::LOADS) {
        oa.issue1(st, wave, s * bf::BK, s < nsteps, i);
      } else {
        const int j = i - bf::LOADS;
        ob.issue1(st + bf::OPER * 2, wave, s < nsteps ? kro[j] + (uint32_t)s * slice_bytes : bf::kOOB, j);
      }
    };
    run_row_mainloop<bf::KC, bf::MNC, WTM>(t.mvalid, nmb, lds, ring, nsteps, issue, acc, wm, wn, lane);
  }
  float* stage = (float*)lds;
  if constexpr (EPI == kEpiStore || EPI == kEpiStoreAct) {
    NoPre none;
    NoPre::Data nd[2];
    const __amdgpu_buffer_rsrc_t rc = tile_rows(P.c, row0, P.ldc, 2);
    const __amdgpu_buffer_rsrc_t rc2 = tile_rows(P.c2, row0, P.ldc2, 2);
    staged_epilogue<WTM>(stage, acc, wm, wn, lane, tid, t.mvalid, none, nd, false, [&](int m, int col, float (&v)[4], NoPre::Data&, int) {
      if (m >= t.mvalid) return;  // uniform per wave
      __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])}, rc,
                                            ((uint32_t)m * (uint32_t)P.ldc + t.n0 + col) * 2u, 0, kEpiNT);
      if constexpr (EPI == kEpiStoreAct) {
        // activation of the stored (rounded) h, the value the backward sees
        float a[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float r = relu(round_t<uint16_t>(v[q]));
          a[q] = r * r;
        }
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])}, rc2,
                                              ((uint32_t)m * (uint32_t)P.ldc2 + t.n0 + col) * 2u, 0, kEpiNT);
      }
    });
  } else {
    dgrad2_epilogue<WTM>(P, t, lds, acc, wm, wn, lane, tid, my_prob);
  }
}


// BMV: tile rows (256, or 192 as two wave rows of 96).  A 256-row tile that
// holds at most 192 rows runs the 96-row wave layout (a choice made per tile
// from its row count; the MFMA order per output element is the same).
template <int BL, int EPI, int BMV>
__global__ __launch_bounds__(256) void rowgemm_bf16_kernel(RowGemmParams P) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[bf::ring_bytes<kRowNS> / 2];
  RowTile t;
  const int kind = row_tile<BMV, bf::BN>(P, t);
  if (kind == kTileSide) dprob_side(P, t.nt);
  if (kind != kTileGemm) return;
  if constexpr (BMV == 256) {
    if (t.mvalid <= kRowTile2)
      rowgemm_bf16_tile<BL, EPI, kRowTile2 / 2>(P, t, lds);
    else
      rowgemm_bf16_tile<BL, EPI, 128>(P, t, lds);
  } else {
    rowgemm_bf16_tile<BL, EPI, BMV / 2>(P, t, lds);
  }
}

// Entries of the gathered-row table past a chunk of klen rows: the main loop
// reads rows up to (ceil(klen / 32) + NS - 2) * 32 - 1 < klen + 128 (the last
// slice and those prefetched past it, NS = 4 slots).
constexpr int kRowoffPad = 160;
static_assert(bf::NSTAGE == 4, "row table padding sized for a 4-slot ring");

// One weight-gradient tile: dW[m0:m0+256, n0:n0+256] of expert t.g over the
// rows of chunk t.s, into dst (dW itself, or a split-K partial slot).
template <bool A_GATHER, bool B_GATHER>
DEV void wgrad_bf16_tile(const WgradParams& P, const WgradTile& t, float* dst, uint16_t* lds, uint32_t* s_rowoff) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t ring = bf::lds_base(lds);
  const int wm = wave >> 1, wn = wave & 1;
  static_assert(A_GATHER != B_GATHER, "exactly one operand is gathered by token");
  const uint32_t ld_gather = (uint32_t)(A_GATHER ? P.lda : P.ldb) * 2u;
  const uint32_t ld_direct = (uint32_t)(A_GATHER ? P.ldb : P.lda) * 2u;
  // Entries past the chunk (read by the loads of its last slice and of the
  // slices prefetched past it) hold kOOB, so those rows read zeros.  Eight
  // entries per thread are loaded before any is stored, so a long chunk
  // waits on one load latency per 2048 rows instead of one per 256.
  // (The loads read a clamped index unconditionally, so that they are not
  // split into branches that each wait for their load.)
  const int nrow = t.klen + kRowoffPad, last = t.klen - 1;
  for (int i0 = 0; i0 < nrow; i0 += 8 * 256) {
    int v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 256 + tid;
      if (i0 + u * 256 < t.klen) v[u] = P.row_tok[t.row0 + (i < t.klen ? i : last)];  // uniform test
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 256 + tid;
      if (i < nrow) s_rowoff[i] = i < t.klen ? (uint32_t)v[u] * ld_gather : bf::kOOB;
    }
  }
  __syncthreads();

  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  // The direct operand (rows of dh or act_p, which can exceed 2 GiB) is
  // addressed from the chunk's first row; the gathered one (x or dy, by
  // token) from its start.
  const void* dbase = row_ptr(A_GATHER ? P.b : P.a, t.row0, A_GATHER ? P.ldb : P.lda, 2);
  const uint32_t dbytes = (uint32_t)t.klen * ld_direct;
  bf::MncOperand oa, ob;
  oa.init(A_GATHER ? P.a : dbase, A_GATHER ? P.a_bytes : dbytes, wave, lane, t.m0);
  ob.init(A_GATHER ? dbase : P.b, A_GATHER ? dbytes : P.b_bytes, wave, lane, t.n0);
  const int nsteps = (t.klen + bf::BK - 1) / bf::BK;
  // Per load j of a slice, this lane's k row is krow(j) + 32 s.  The direct
  // operand's row offset advances by a scalar per slice, and its rows past
  // the chunk lie past the buffer's num_records (the chunk's own rows), so
  // they read zeros; the gathered operand's offsets of slice s+1 are read
  // from LDS right after slice s is issued, so an issue never waits on that
  // read.
  uint32_t dir[bf::LOADS], gat[bf::LOADS];
  int kr[bf::LOADS];
#pragma unroll
  for (int j = 0; j < bf::LOADS; ++j) {
    kr[j] = bf::MncOperand::krow(wave, lane, j);
    dir[j] = (uint32_t)kr[j] * ld_direct;
  }
  auto fetch = [&](int s) {
#pragma unroll
    for (int j = 0; j < bf::LOADS; ++j) gat[j] = s_rowoff[s * bf::BK + kr[j]];
  };
  fetch(0);
  const uint32_t dir_step = (uint32_t)bf::BK * ld_direct;
  bf::mainloop<bf::MNC, bf::MNC, 4, bf::NSTAGE, 128, true>(lds, ring, nsteps, [&](int s, uint32_t st, int i) {
    const int j = i & (bf::LOADS - 1);
    const uint32_t d = dir[j] + (uint32_t)s * dir_step;
    if (i < bf::LOADS)
      oa.issue1(st, wave, A_GATHER ? gat[j] : d, j);
    else
      ob.issue1(st + bf::OPER * 2, wave, B_GATHER ? gat[j] : d, j);
    if (i == 2 * bf::LOADS - 1) fetch(s + 1);
  }, acc, wm, wn, lane);
  NoPre none;
  const __amdgpu_buffer_rsrc_t rd = buf(dst);
  NoPre::Data nd[2];
  auto offset = [&](int m, int col) { return ((uint32_t)(t.m0 + m) * (uint32_t)P.N + t.n0 + col) * 4u; };
  // two instantiations, so that the store loop carries no per-store branch
  if (P.atomic && t.S > 1) {
    staged_epilogue((float*)lds, acc, wm, wn, lane, tid, bf::BM, none, nd, false, [&](int m, int col, float (&v)[4], NoPre::Data&, int) {
      float* po = dst + offset(m, col) / 4u;
#pragma unroll
      for (int q = 0; q < 4; ++q) atomicAdd(po + q, v[q]);
    });
  } else {
    staged_epilogue((float*)lds, acc, wm, wn, lane, tid, bf::BM, none, nd, false, [&](int m, int col, float (&v)[4], NoPre::Data&, int) {
      __builtin_amdgcn_raw_buffer_store_b128(f32x4_t{v[0], v[1], v[2], v[3]}, rd, offset(m, col), 0, kEpiNT);
    });
  }
}

// Ordered split-K reduction of one dW tile, run by the chunk that finishes
// last (deterministic mode).  Every chunk of a split expert has stored its
// partial tile (chunk 0 into dW itself, chunk s >= 1 into slot
// first_slot + s - 1), made the stores visible at device scope and taken an
// integer ticket for the tile; integer addition is exact, so the ticket
// count does not depend on arrival order, and the chunk that takes the last
// ticket adds the partials in chunk order:
//   dW = ((part_0 + part_1) + part_2) + ... + part_{S-1}
// Which workgroup does the adding changes nothing in the sum.  No workgroup
// waits on another, and the tickets were zeroed by the prologue launch.
DEV void wgrad_ordered_tail(const WgradParams& P, const WgradTile& t, int S, int first_slot, int tile, int tiles,
                            int* s_flag) {
  __threadfence();  // release this workgroup's partial stores
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = atomicAdd(P.tickets + (int64_t)first_slot * tiles + tile, 1);
    s_flag[0] = old == S - 1;
  }
  __syncthreads();
  if (!s_flag[0]) return;
  __threadfence();  // acquire the other chunks' partials
  const int64_t MN = (int64_t)P.M * P.N;
  float* out = P.dw + (int64_t)t.g * MN;
  const float* sl = P.slots + (int64_t)first_slot * MN;
  // 256 x 256 floats: thread tid adds 4 consecutive columns of 64 rows
#pragma unroll 4
  for (int q = 0; q < 64; ++q) {
    const int m = q * 4 + (threadIdx.x >> 6);
    const int64_t o = (int64_t)(t.m0 + m) * P.N + t.n0 + 4 * (threadIdx.x & 63);
    f32x4_t v = *(const f32x4_t*)(out + o);
    for (int s = 1; s < S; ++s) {
      const f32x4_t w = *(const f32x4_t*)(sl + (int64_t)(s - 1) * MN + o);
      v[0] = v[0] + w[0];
      v[1] = v[1] + w[1];
      v[2] = v[2] + w[2];
      v[3] = v[3] + w[3];
    }
    *(f32x4_t*)(out + o) = v;
  }
}

// Unit L of one of the two weight gradients of the paired launch: tile
// L % tiles of weight-gradient unit L / tiles of the routing work list.
template <bool A_GATHER, bool B_GATHER>
DEV void wgrad_pair_unit(const WgradParams& P, int64_t L, int tiles, uint16_t* lds, uint32_t* s_rowoff) {
  const int nN = P.N / bf::BN;
  const int64_t u = (uint32_t)L / (uint32_t)tiles;  // L < 2^31 (one unit per workgroup)
  const int tile = (int)((uint32_t)L % (uint32_t)tiles);
  const int4 en = ((const int4*)(P.units + P.units_at))[u];
  WgradTile t;
  t.g = __builtin_amdgcn_readfirstlane(en.x & 0x3fffffff);
  t.S = (en.x >> 30) ? 2 : 1;  // only "split or not" matters here
  t.s = 0;
  t.row0 = (int64_t)__builtin_amdgcn_readfirstlane(en.y);
  t.klen = __builtin_amdgcn_readfirstlane(en.z);
  const int slot = __builtin_amdgcn_readfirstlane(en.w);
  t.m0 = (tile / nN) * bf::BM;
  t.n0 = (tile % nN) * bf::BN;
  float* dst = (!P.atomic && slot >= 0) ? P.slots + (int64_t)slot * P.M * P.N : P.dw + (int64_t)t.g * P.M * P.N;
  wgrad_bf16_tile<A_GATHER, B_GATHER>(P, t, dst, lds, s_rowoff);
  if (!P.atomic && t.S > 1) {
    const int4 ax = ((const int4*)(P.units + P.aux_at))[u];   // {S, chunk, first slot, 0}
    wgrad_ordered_tail(P, t, __builtin_amdgcn_readfirstlane(ax.x), __builtin_amdgcn_readfirstlane(ax.z), tile,
                       tiles, (int*)lds);
  }
}

// Both weight gradients in one launch: units [0, U1) are dW1 tiles (rows of
// x gathered by token, dh rows), [U1, U1 + U2) dW2 tiles (act_p rows, dy
// gathered by token), over the (expert, K chunk) units of the routing work
// list.
__global__ __launch_bounds__(256) void wgrad_pair_bf16_kernel(WgradParams P1, WgradParams P2, int ncu) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[bf::LDS_BYTES / 2];
  __shared__ uint32_t s_rowoff[kMaxChunkRows + kRowoffPad];  // byte offset of each gathered row of the chunk
  const int tiles1 = (P1.M / bf::BM) * (P1.N / bf::BN), tiles2 = (P2.M / bf::BM) * (P2.N / bf::BN);
  const int64_t units = P1.units[1];
  const int64_t U1 = units * tiles1, U2 = units * tiles2;
  const int64_t L = map_unit_rounds(blockIdx.x, U1 + U2, ncu, P1.seed);
  if (L < 0) return;
  if (L >= U1)
    wgrad_pair_unit<false, true>(P2, L - U1, tiles2, lds, s_rowoff);
  else
    wgrad_pair_unit<true, false>(P1, L, tiles1, lds, s_rowoff);
}

// ================================================================ MXFP8
// Grouped row GEMM on MXFP8 operands (OCP MX v1.0: E4M3 codes, an E8M0 scale
// per 32 consecutive k): C[r, n] = sum_k A[r, k] B_g[n, k] with both operands
// K-contiguous (rows of codes, scales [rows][K/32]), through
// v_mfma_scale_f32_32x32x64_f8f6f4; output bf16 rows.  A K slice is 64
// codes, so a tile row of a slice is 64 bytes and the DMA loaders and the LDS
// layout of the bf16 K-contiguous tiles carry over unchanged.  Lane layout of
// the scaled MFMA (gfx950): lane l = 32h + i holds, for row i, the codes of k
// = 16h .. 16h+15 in bytes 0..15 and k = 32+16h .. 32+16h+15 in bytes
// 16..31, i.e. chunks h and 2+h of the row; the scale register of lane
// 32kb + i carries the E8M0 byte of row i, k-block kb.  Each tile's scales
// (up to 256 rows x K/32 bytes per operand) are staged in LDS before the main
// loop.
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t_ __attribute__((ext_vector_type(4)));

struct MxFrags {
  i32x8_t a[4], b[4];
  int sa[4], sb[4];
};

DEV void mx_read_block(const uint8_t* op, const uint8_t* scales, int nkb, int kb, int row, int h, i32x8_t& f,
                       int& sc) {
  const int sw = bf::kc_swz(row);
  const i32x4_t_ lo = *(const i32x4_t_*)(op + row * 64 + ((h ^ sw) << 4));
  const i32x4_t_ hi = *(const i32x4_t_*)(op + row * 64 + (((2 + h) ^ sw) << 4));
  f = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  sc = scales[row * nkb + (kb < nkb ? kb : nkb - 1)];
}

// E8M0 scales of an MXFP8 operand pair streamed through LDS with the codes,
// for operands whose scales are laid out slice-major ([slices][rows][2]: the
// two 32-code block scales of each row in each 64-code slice), so that the
// 512 bytes of a 256-row tile's slice are contiguous.  Each wave issues one
// 16-byte DMA per slice: wave 0 the A scales and wave 1 the B scales (lanes
// 0..31), every other lane and wave a load past the buffer end, whose zeros
// land in the wave's own KiB of the slot.  Slot layout: A scales at 0 (row
// r: bytes 2r, 2r + 1), B scales at 1024.
constexpr int kMxScaleSlot = 4096;
struct MxRingScales {
  bf::i32x4_t rs;
  uint32_t voff;     // byte offset of this lane's 16 bytes of slice 0, or kOOB
  uint32_t sstride;  // bytes per slice of the operand this wave loads
  DEV void init(int wave, int lane, const uint8_t* a, uint32_t a_bytes, uint32_t a_off, uint32_t a_stride,
                const uint8_t* b, uint32_t b_bytes, uint32_t b_off, uint32_t b_stride) {
    const bool is_b = wave == 1;
    rs = bf::make_rsrc(is_b ? b : a, is_b ? b_bytes : a_bytes);
    sstride = is_b ? b_stride : a_stride;
    voff = (wave < 2 && lane < 32) ? (is_b ? b_off : a_off) + (uint32_t)lane * 16u : bf::kOOB;
  }
  DEV void issue(uint32_t slot, int wave, int s, bool live) const {
    bf::dma16(rs, slot + (uint32_t)wave * 1024u, live ? voff : bf::kOOB, live ? (uint32_t)s * sstride : 0u);
  }
};

// Pipelined MXFP8 main loop of one 256-column tile over nsteps slices of 64
// codes (nsteps even), accumulated into acc in a fixed order: slice by
// slice, and within a slice A block by A block against B blocks 0..3.
// Slices at or past nlive load as zeros; slice s of an operand starts
// (kslice0 + s) * a_sstride (b_sstride) bytes past its tile rows' offsets:
// 64 for codes stored K-contiguous, rows * 64 for slice-major codes.
// Scales, RS == false: the scale of tile row r and 32-code block kb of the
// call is s_sa[r * nkb + kb] (s_sb for B; kb past nkb - 1 reads nkb - 1,
// and every byte read must be a finite scale); store_scales() writes those
// LDS arrays from registers the caller loaded before the call: it runs
// once the loads of slices 0..2 have been issued and every load issued
// before them has landed.  RS == true: the scales come through the ring
// (MxRingScales rsc, 4 slots of kMxScaleSlot bytes at s_sa), slice
// kslice0 + s with the codes of slice s.
// On return loads past the last slice may still be in flight and other
// waves may still read LDS: the caller drains and synchronises before
// reusing it.
template <int NA, int WTM, bool RS, class StoreScales>
DEV void mx_mainloop(uint16_t* lds, const bf::KcOperand& oa, const bf::KcOperand& ob, uint32_t a_sstride,
                     uint32_t b_sstride, const MxRingScales& rsc, int kslice0, int nsteps, int nlive,
                     const uint8_t* s_sa, const uint8_t* s_sb, int nkb, StoreScales store_scales,
                     f32x16_t (&acc)[4][4], int wave, int lane, int wm, int wn) {
  const uint32_t ring = bf::lds_base(lds);
  const uint32_t sring = bf::lds_base(s_sa);
  constexpr int NL = RS ? 9 : 8;   // loads per slice and thread
  // slice s: 64 codes = 64 bytes per row, the size of a bf16 slice of 32
  // With RS the operands are slice-major and their buffers end after slice
  // nlive - 1, so a slice past it lies past num_records and reads zeros with
  // no per-load select; K-contiguous rows would run into the next row.
  auto issue = [&](int s, int i) __attribute__((always_inline)) {
    const uint32_t st = ring + (uint32_t)(s & 3) * (bf::STAGE * 2);
    const bool live = RS || s < nlive;
    if (i < bf::LOADS)
      oa.issue1_bytes(st, wave, (uint32_t)(kslice0 + s) * a_sstride, live, i);
    else if (i < 2 * bf::LOADS)
      ob.issue1_bytes(st + bf::OPER * 2, wave, (uint32_t)(kslice0 + s) * b_sstride, live, i - bf::LOADS);
    else
      rsc.issue(sring + (uint32_t)(s & 3) * kMxScaleSlot, wave, kslice0 + s, live);
  };
  const int h = lane >> 5, r32 = lane & 31;
  auto slot = [&](int s) { return (const uint8_t*)(lds + (s & 3) * bf::STAGE); };
  auto read = [&](MxFrags& f, int s, auto G) __attribute__((always_inline)) {   // group G: A block G (G < 4) or B block G-4
    constexpr int g = decltype(G)::value;
    const uint8_t* st = slot(s);
    if constexpr (RS) {
      const uint8_t* ss = s_sa + (s & 3) * kMxScaleSlot;
      if constexpr (g < NA)
        mx_read_block(st, ss, 2, h, wm * WTM + g * 32 + r32, h, f.a[g], f.sa[g]);
      else if constexpr (g >= 4)
        mx_read_block(st + bf::OPER * 2, ss + 1024, 2, h, wn * 128 + (g - 4) * 32 + r32, h, f.b[g - 4], f.sb[g - 4]);
    } else {
      if constexpr (g < NA)
        mx_read_block(st, s_sa, nkb, 2 * s + h, wm * WTM + g * 32 + r32, h, f.a[g], f.sa[g]);
      else if constexpr (g >= 4)
        mx_read_block(st + bf::OPER * 2, s_sb, nkb, 2 * s + h, wn * 128 + (g - 4) * 32 + r32, h, f.b[g - 4],
                      f.sb[g - 4]);
    }
  };
  // A block mb of fa against the four B blocks of fb; the tile's first slice
  // (FIRST) takes a zero accumulator input instead of zeroed registers
  auto mma = [&](const MxFrags& fa, const MxFrags& fb, auto MB, auto FIRST) __attribute__((always_inline)) {
    constexpr int mb = decltype(MB)::value;
    constexpr bool first = decltype(FIRST)::value;
    if constexpr (mb >= NA) return;
    const f32x16_t zero = {};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb.b[j], fa.a[mb], first ? zero : acc[mb][j], 0, 0, 0,
                                                                   fb.sb[j], 0, fa.sa[mb]);
  };
  // prologue: slices 0..2 in flight; the scale words (loaded before them)
  // stored; slice 0 landed and the stores done in every wave; B blocks read
#pragma unroll
  for (int s = 0; s < 3; ++s)
#pragma unroll
    for (int i = 0; i < NL; ++i) issue(s, i);
  if constexpr (RS) {
    asm volatile("s_waitcnt vmcnt(18)\n\ts_barrier" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
    store_scales();
    asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  MxFrags f, g;      // f.a: A blocks of the current slice; f.b and g.b: B blocks, alternating by step
  read(f, 0, std::integral_constant<int, 4>{});
  read(f, 0, std::integral_constant<int, 5>{});
  read(f, 0, std::integral_constant<int, 6>{});
  read(f, 0, std::integral_constant<int, 7>{});
  // step s: slice s+1 landed and every wave is done with slice s-1, whose slot
  // takes slice s+3.  The A blocks of slice s are read one ahead of their
  // MFMAs; the B blocks of slice s+1 (past the last slice: zero codes and a
  // clamped scale index, never multiplied) are read into the other B set in
  // between, so the sets swap roles each step and nothing is copied.
  auto step = [&](int s, const MxFrags& bcur, MxFrags& bnext, auto first) __attribute__((always_inline)) {
    if constexpr (RS)
      asm volatile("s_waitcnt vmcnt(9) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    read(f, s, std::integral_constant<int, 0>{});
    issue(s + 3, 0);
    read(f, s, std::integral_constant<int, 1>{});
    issue(s + 3, 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(f, bcur, std::integral_constant<int, 0>{}, first);
    read(bnext, s + 1, std::integral_constant<int, 4>{});
    read(f, s, std::integral_constant<int, 2>{});
    issue(s + 3, 2);
    issue(s + 3, 3);
    __builtin_amdgcn_sched_barrier(0);
    mma(f, bcur, std::integral_constant<int, 1>{}, first);
    read(bnext, s + 1, std::integral_constant<int, 5>{});
    read(f, s, std::integral_constant<int, 3>{});
    issue(s + 3, 4);
    issue(s + 3, 5);
    __builtin_amdgcn_sched_barrier(0);
    mma(f, bcur, std::integral_constant<int, 2>{}, first);
    read(bnext, s + 1, std::integral_constant<int, 6>{});
    read(bnext, s + 1, std::integral_constant<int, 7>{});
    issue(s + 3, 6);
    issue(s + 3, 7);
    if constexpr (RS) issue(s + 3, 8);
    __builtin_amdgcn_sched_barrier(0);
    mma(f, bcur, std::integral_constant<int, 3>{}, first);
    __builtin_amdgcn_sched_barrier(0);
  };
  if (nsteps <= 0) return;
  step(0, f, g, std::true_type{});
  step(1, g, f, std::false_type{});
#pragma unroll 1
  for (int s = 2; s < nsteps; s += 2) {
    step(s, f, g, std::false_type{});
    step(s + 1, g, f, std::false_type{});
  }
}

// BMV: tile rows (256, or 192 as two wave rows of 96: NA = 3 A blocks a
// wave).  EPI: kEpiStore (bf16 rows of C), kEpiStoreAct (also relu(C)^2 of
// the rounded C, into c2) or kEpiDgrad2 (the fc2 dgrad epilogue on G = C).  With P.a_rows, A row r is row a_rows[r] of the codes
// and of the scales (the fc2 dgrad gathers dy by token).
static_assert(kProbOff + bf::BM * 4 <= bf::LDS_BYTES, "fc2 dgrad epilogue scratch must fit in the MXFP8 ring");
template <int BMV, int EPI>
__global__ __launch_bounds__(256) void mx_rowgemm_kernel(RowGemmParams P) {
  constexpr int WTM = BMV / 2, NA = WTM / 32;
  __shared__ __attribute__((aligned(16))) uint16_t lds[bf::LDS_BYTES / 2];
  __shared__ __attribute__((aligned(16))) uint8_t s_sa[256 * (kMxMaxK / 32)];
  __shared__ __attribute__((aligned(16))) uint8_t s_sb[256 * (kMxMaxK / 32)];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  RowTile t;
  if (row_tile<BMV, bf::BN>(P, t) != kTileGemm) return;
  float my_prob = 0.f;
  if constexpr (EPI == kEpiDgrad2) my_prob = tid < t.mvalid ? P.row_prob[t.off + t.m0 + tid] : 0.f;
  const int nkb = P.K / 32;
  const int64_t sg = (int64_t)t.g * P.b_sgstride;
  auto arow = [&](int r) -> int64_t {   // source row of tile row r < t.mvalid
    return P.a_rows ? (int64_t)P.a_rows[t.off + t.m0 + r] : t.off + t.m0 + r;
  };
  // the tile's scales, 4-byte words, all loads issued up front (rows past the
  // tile's valid rows read row 0 of the tile: their codes load as zeros); they
  // are stored to LDS once the slice prologue has been issued
  constexpr int kSw = 256 * (kMxMaxK / 32) / 4 / 256;   // words per thread and operand, at most
  const int nw = 256 * (nkb / 4);
  uint32_t wa[kSw], wb[kSw];
#pragma unroll
  for (int q = 0; q < kSw; ++q) {
    const int idx = tid + 256 * q;
    const int r = idx / (nkb / 4), c = idx % (nkb / 4);
    const int ra = r < t.mvalid ? r : 0;
    wa[q] = idx < nw ? ((const uint32_t*)(P.a_scales + arow(ra) * nkb))[c] : 0u;
    wb[q] = idx < nw ? ((const uint32_t*)(P.b_scales + sg + (int64_t)(t.n0 + (idx < nw ? r : 0)) * nkb))[c] : 0u;
  }
  // codes gathered by token from the start of a[T][lda]; otherwise the
  // tile's own rows from the first (arrays of routed rows can exceed 2 GiB)
  const bool gathered = P.a_rows != nullptr;
  const int64_t row0 = t.off + t.m0;
  bf::KcOperand oa, ob;
  oa.init(gathered ? P.a : row_ptr(P.a, row0, P.lda, 1), gathered ? P.a_bytes : (uint32_t)(t.mvalid * P.lda), wave,
          lane, [&](int r) -> uint32_t {   // branch-free, as in the bf16 kernel
    const int64_t row = arow(r < t.mvalid ? r : t.mvalid - 1);
    return r < t.mvalid ? (uint32_t)((gathered ? row : row - row0) * P.lda) : bf::kOOB;
  });
  ob.init((const uint8_t*)P.b + (int64_t)t.g * P.b_gstride, P.b_bytes, wave, lane,
          [&](int r) -> uint32_t { return (uint32_t)((t.n0 + r) * P.ldb); });
  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  // the number of slices is even (K is a multiple of 128)
  const int nsteps = P.K / 64;
  __builtin_assume(nsteps > 0);  // K is a positive multiple of 128 (checked at the boundary)
  const MxRingScales none{};
  mx_mainloop<NA, WTM, false>(lds, oa, ob, 64u, 64u, none, 0, nsteps, nsteps, s_sa, s_sb, nkb, [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < kSw; ++q) {
      const int idx = tid + 256 * q;
      if (idx < nw) {
        ((uint32_t*)s_sa)[idx] = wa[q];
        ((uint32_t*)s_sb)[idx] = wb[q];
      }
    }
  }, acc, wave, lane, wm, wn);
  bf::block_barrier();
  if constexpr (EPI == kEpiDgrad2) {
    dgrad2_epilogue<WTM>(P, t, lds, acc, wm, wn, lane, tid, my_prob);
  } else {
    float* stage = (float*)lds;
    NoPre none;
    NoPre::Data nd[2];
    const __amdgpu_buffer_rsrc_t rc = tile_rows(P.c, row0, P.ldc, 2);
    const __amdgpu_buffer_rsrc_t rc2 = tile_rows(P.c2, row0, P.ldc2, 2);
    staged_epilogue<WTM>(stage, acc, wm, wn, lane, tid, t.mvalid, none, nd, false, [&](int m, int col, float (&v)[4], NoPre::Data&, int) {
      if (m >= t.mvalid) return;  // uniform per wave
      __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])}, rc,
                                            ((uint32_t)m * (uint32_t)P.ldc + t.n0 + col) * 2u, 0, kEpiNT);
      if constexpr (EPI == kEpiStoreAct) {
        // activation of the stored (rounded) h, as in the bf16 forward
        float a[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float r = relu(round_t<uint16_t>(v[q]));
          a[q] = r * r;
        }
        __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])}, rc2,
                                              ((uint32_t)m * (uint32_t)P.ldc2 + t.n0 + col) * 2u, 0, kEpiNT);
      }
    });
  }
}

// MXFP8 weight gradients, both matrices in one launch.  Unit (g, matrix,
// 256x256 tile): dW1_g tiles take A = X^T codes (rows over d_model) and
// B = dH^T codes (rows over d_ffn), dW2_g tiles A = act^T and B = dY^T; K
// runs over the expert's padded routed rows, whose count is even in 64-code
// slices or completed by one slice of zeros.  One workgroup accumulates a
// tile over the whole K range in slice order and stores it once, so the
// result does not depend on the launch order and needs no reduction.  Codes
// and scales are slice-major (a tile's slice is one contiguous run of 16 KiB
// of codes and 512 bytes of scales); the scales stream through LDS with the
// codes.  An expert without rows gets a zero tile.
template <class T>
DEV T pick(int c, T a, T b) {
  return c ? a : b;
}
__global__ __launch_bounds__(256) void mx_wgrad_kernel(MxWgradParams P) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[bf::LDS_BYTES / 2];
  __shared__ __attribute__((aligned(16))) uint8_t s_sc[4 * kMxScaleSlot];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles = (P.D / 256) * (P.F / 256);
  const int64_t L = map_unit(blockIdx.x, (int64_t)P.groups * 2 * tiles, P.seed);
  if (L < 0) return;
  const uint32_t Lu = (uint32_t)L;  // L < 2^31 (one unit per workgroup)
  const int g = (int)(Lu / (2u * tiles)), mat = (int)(Lu / (uint32_t)tiles) & 1, tile = (int)(Lu % (uint32_t)tiles);
  // selections on copies: a conditional over two members of the kernel
  // argument is an lvalue and would move the argument to scratch
  const int M = pick(mat, P.F, P.D), N = pick(mat, P.D, P.F);
  const int m0 = (tile / (N / 256)) * 256, n0 = (tile % (N / 256)) * 256;
  const uint8_t* ac = pick(mat, P.act_codes, P.x_codes);
  const uint8_t* as = pick(mat, P.act_scales, P.x_scales);
  const uint8_t* bc = pick(mat, P.dy_codes, P.dh_codes);
  const uint8_t* bs = pick(mat, P.dy_scales, P.dh_scales);
  float* dst = pick(mat, P.dw2, P.dw1) + (int64_t)g * P.D * P.F;
  const int p0 = P.poff[g], nsl = (P.poff[g + 1] - p0) / 64;
  // slice-major codes: slice j of operand rows R at byte (j R + row) 64,
  // addressed from the expert's first slice (the encodings of all routed
  // rows can exceed 2 GiB; one expert's, at most T rows, stay below 2^31
  // bytes, which the host checks)
  const int64_t j0 = p0 / 64;
  bf::KcOperand oa, ob;
  oa.init(ac + j0 * M * 64, (uint32_t)(nsl * M * 64), wave, lane,
          [&](int r) -> uint32_t { return (uint32_t)((m0 + r) * 64); });
  ob.init(bc + j0 * N * 64, (uint32_t)(nsl * N * 64), wave, lane,
          [&](int r) -> uint32_t { return (uint32_t)((n0 + r) * 64); });
  // slice-major scales: slice j of operand rows R at byte (j R + row) 2
  MxRingScales rsc;
  rsc.init(wave, lane, as + j0 * M * 2, (uint32_t)(nsl * M * 2), (uint32_t)(m0 * 2), (uint32_t)(2 * M),
           bs + j0 * N * 2, (uint32_t)(nsl * N * 2), (uint32_t)(n0 * 2), (uint32_t)(2 * N));
  f32x16_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  mx_mainloop<4, 128, true>(lds, oa, ob, (uint32_t)(64 * M), (uint32_t)(64 * N), rsc, 0, (nsl + 1) & ~1, nsl, s_sc,
                            s_sc, 2, [] {}, acc, wave, lane, wm, wn);
  // every load (those of the zero slices past the end included) landed and
  // every wave done with the ring before the epilogue stages through it
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  bf::block_barrier();
  NoPre none;
  NoPre::Data nd[2];
  const __amdgpu_buffer_rsrc_t rd = buf(dst);
  staged_epilogue((float*)lds, acc, wm, wn, lane, tid, bf::BM, none, nd, false, [&](int m, int col, float (&v)[4], NoPre::Data&, int) {
    const uint32_t o = ((uint32_t)(m0 + m) * (uint32_t)N + n0 + col) * 4u;
    __builtin_amdgcn_raw_buffer_store_b128(f32x4_t{v[0], v[1], v[2], v[3]}, rd, o, 0, kEpiNT);
  });
}

hipError_t launch_mx_wgrad(const MxWgradParams& P, hipStream_t st) {
  const int64_t units = (int64_t)P.groups * 2 * (P.D / 256) * (P.F / 256);
  if (units == 0) return hipSuccess;
  mx_wgrad_kernel<<<grid_for_units(units), 256, 0, st>>>(P);
  return hipGetLastError();
}

// ================================================================= fp32
template <bool B_MNC, int EPI>
__global__ __launch_bounds__(256) void rowgemm_f32_kernel(RowGemmParams P) {
  __shared__ __attribute__((aligned(16))) float lds[f32::LDS_BYTES / 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  RowTile t;
  const int kind = row_tile<f32::BM, f32::BN>(P, t);
  if (kind == kTileSide) dprob_side(P, t.nt);
  if (kind != kTileGemm) return;
  float* As0 = lds;
  float* Bs0 = lds + 2 * f32::OPER;
  f32::KcLoader la;
  la.init(tid, (const float*)P.a, P.lda, P.a_rows, t.off + t.m0, t.mvalid);
  const float* Bg = (const float*)P.b + (int64_t)t.g * P.b_gstride;
  f32x16_t acc[1][1];
  f32::zero_acc(acc[0][0]);
  const int nsteps = P.K / f32::BK;
  f32::KcLoader lbk;
  f32::MncLoader lbm;
  if (!B_MNC) lbk.init(tid, Bg, P.ldb, nullptr, t.n0, f32::BN);
  auto loadB = [&](int s) {
    if constexpr (B_MNC)
      lbm.load(tid, [&](int k) { return Bg + ((int64_t)s * f32::BK + k) * P.ldb + t.n0; });
    else
      lbk.load((int64_t)s * f32::BK);
  };
  auto storeB = [&](float* dst) {
    if constexpr (B_MNC)
      lbm.store(dst, tid);
    else
      lbk.store(dst, tid);
  };
  la.load(0);
  loadB(0);
  la.store(As0, tid);
  storeB(Bs0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int cur = s & 1;
    if (s + 1 < nsteps) {
      la.load((int64_t)(s + 1) * f32::BK);
      loadB(s + 1);
    }
    f32::mma_slice(As0 + cur * f32::OPER, Bs0 + cur * f32::OPER, acc[0][0], wm, wn, lane);
    if (s + 1 < nsteps) {
      la.store(As0 + (cur ^ 1) * f32::OPER, tid);
      storeB(Bs0 + (cur ^ 1) * f32::OPER);
    }
    __syncthreads();
  }
  row_epilogue<float, 1, 1, 32, 32, f32::BM, 2, EPI>(P, t, acc, lds, wm, wn, lane, tid);
}

template <bool A_GATHER, bool B_GATHER>
__global__ __launch_bounds__(256) void wgrad_f32_kernel(WgradParams P) {
  __shared__ __attribute__((aligned(16))) float lds[f32::LDS_BYTES / 4];
  __shared__ int s_tok[kMaxChunkRows];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  WgradTile t;
  if (!wgrad_tile<f32::BM, f32::BN>(P, t)) return;
  for (int i = tid; i < t.klen; i += 256) s_tok[i] = P.row_tok[t.row0 + i];
  __syncthreads();
  float* As0 = lds;
  float* Bs0 = lds + 2 * f32::OPER;
  f32x16_t acc[1][1];
  f32::zero_acc(acc[0][0]);
  const int nsteps = (t.klen + f32::BK - 1) / f32::BK;
  f32::MncLoader la, lb;
  const float* Ab = (const float*)P.a;
  const float* Bb = (const float*)P.b;
  auto rows = [&](int st, const float* base, bool gather, int64_t ld, int mn0) {
    return [=, &t](int k) -> const float* {
      const int kk = st * f32::BK + k;
      if (kk >= t.klen) return nullptr;
      const int64_t r = gather ? (int64_t)s_tok[kk] : t.row0 + kk;
      return base + r * ld + mn0;
    };
  };
  if (nsteps > 0) {
    la.load(tid, rows(0, Ab, A_GATHER, P.lda, t.m0));
    lb.load(tid, rows(0, Bb, B_GATHER, P.ldb, t.n0));
    la.store(As0, tid);
    lb.store(Bs0, tid);
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
      const int cur = st & 1;
      if (st + 1 < nsteps) {
        la.load(tid, rows(st + 1, Ab, A_GATHER, P.lda, t.m0));
        lb.load(tid, rows(st + 1, Bb, B_GATHER, P.ldb, t.n0));
      }
      f32::mma_slice(As0 + cur * f32::OPER, Bs0 + cur * f32::OPER, acc[0][0], wm, wn, lane);
      if (st + 1 < nsteps) {
        la.store(As0 + (cur ^ 1) * f32::OPER, tid);
        lb.store(Bs0 + (cur ^ 1) * f32::OPER, tid);
      }
      __syncthreads();
    }
  }
  wgrad_store<1, 1, 32, 32>(wgrad_dst(P, t), P.N, P.atomic && t.S > 1, t.m0, t.n0, acc, wm, wn, lane);
}

// ============================================================ prep/reduce
// Prologue of moe_bwd_wgrad.
//  * act_p = p * relu(h)^2 for every routed row r < R (R = offsets[G]), in
//    the same float32 steps as the forward's activation: rh = max(h, 0),
//    a = rh * rh, act_p = RNE(p * a);
//  * block 0, float32 path only: unit_start[g] = sum_{g'<g} S_g' and
//    slot_base[g] = sum_{g'<g} (S_g' - 1), S_g = max(1, ceil(cnt_g / kc));
//  * the arrival tickets of the split tiles are zeroed;
//  * atomic mode zeroes dW of every split expert (S_g >= 2), whose chunks
//    then add into it.
template <typename T>
__global__ __launch_bounds__(256) void wgrad_prep_kernel(WgradPrepParams P) {
  __shared__ int s_pre[kMaxExperts + 1];
  __shared__ int s_tmp[8];
  const int G = P.groups;
  auto nsplit = [&](int g) {
    const int c = P.counts[g];
    return c > P.kc ? (c + P.kc - 1) / P.kc : 1;
  };
  if (P.sched && blockIdx.x == 0) {
    block_exclusive_scan<256>(s_pre, s_tmp, G, nsplit);
    for (int g = threadIdx.x; g <= G; g += 256) P.sched[g] = s_pre[g];
    __syncthreads();
    block_exclusive_scan<256>(s_pre, s_tmp, G, [&](int g) { return nsplit(g) - 1; });
    for (int g = threadIdx.x; g <= G; g += 256) P.sched[G + 1 + g] = s_pre[g];
  }
  const int64_t gtid = (int64_t)blockIdx.x * 256 + threadIdx.x, gstride = (int64_t)gridDim.x * 256;
  for (int64_t i = gtid; i < P.n_tickets; i += gstride) P.tickets[i] = 0;
  // R * N elements of the storage type are below 2^35 bytes (validated on
  // the host), so the number of 16-byte vectors fits 32 bits; element
  // offsets are 64-bit
  constexpr int V = 16 / sizeof(T);
  const int per_row = P.N / V;
  const int nvec = P.offsets[G] * per_row;
  for (int v = (int)gtid; v < nvec; v += (int)gstride) {
    const int r = v / per_row;
    const int64_t e0 = (int64_t)v * V;
    const float p = P.row_prob[r];
    float hv[V], a[V];
    if constexpr (sizeof(T) == 2) {
      const u32x4_t x = __builtin_nontemporal_load((const u32x4_t*)((const uint16_t*)P.h + e0));
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        hv[2 * w] = bf16_to_f32(x[w] & 0xffffu);
        hv[2 * w + 1] = bf16_to_f32(x[w] >> 16);
      }
    } else {
      const f32x4_t x = __builtin_nontemporal_load((const f32x4_t*)((const float*)P.h + e0));
#pragma unroll
      for (int q = 0; q < 4; ++q) hv[q] = x[q];
    }
#pragma unroll
    for (int q = 0; q < V; ++q) {
      const float rh = relu(hv[q]);
      a[q] = p * (rh * rh);
    }
    if constexpr (sizeof(T) == 2) {
      *(u32x4_t*)((uint16_t*)P.act_p + e0) =
          u32x4_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(a[4], a[5]), pack_bf16x2(a[6], a[7])};
    } else {
      *(f32x4_t*)((float*)P.act_p + e0) = f32x4_t{a[0], a[1], a[2], a[3]};
    }
  }
  if (P.atomic) {
    const int64_t per = (int64_t)P.M * P.N / 4;
    for (int g = 0; g < G; ++g) {
      if (nsplit(g) < 2) continue;
      f32x4_t* d1 = (f32x4_t*)(P.dw1 + (int64_t)g * P.M * P.N);
      f32x4_t* d2 = (f32x4_t*)(P.dw2 + (int64_t)g * P.M * P.N);
      for (int64_t i = gtid; i < per; i += gstride) {
        d1[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        d2[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
}

// Ordered split-K reduction (deterministic mode):
//   dW_g = ((part_0 + part_1) + part_2) + ... + part_{S-1}
// part_0 sits in dW_g itself, part_s (s >= 1) in slot slot_base[g] + s - 1.
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(WgradPrepParams P) {
  __shared__ int slot_base[kMaxExperts + 1];  // sum over earlier experts of S - 1
  __shared__ int s_tmp[8];
  const int G = P.groups;
  block_exclusive_scan<256>(slot_base, s_tmp, G, [&](int g) {
    const int c = P.counts[g];
    return c > P.kc ? (c + P.kc - 1) / P.kc - 1 : 0;
  });
  const int64_t MN = (int64_t)P.M * P.N;
  const int64_t per = MN / 4;
  for (int g = 0; g < G; ++g) {
    const int c = P.counts[g];
    const int S = c > P.kc ? (c + P.kc - 1) / P.kc : 1;
    if (S < 2) continue;
    for (int which = 0; which < 2; ++which) {
      f32x4_t* d = (f32x4_t*)((which ? P.dw2 : P.dw1) + g * MN);
      const float* sl = (which ? P.slots2 : P.slots1) + (int64_t)slot_base[g] * MN;
      for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < per; i += (int64_t)gridDim.x * 256) {
        f32x4_t v = d[i];
        for (int s = 1; s < S; ++s) {
          f32x4_t q = *((const f32x4_t*)(sl + (int64_t)(s - 1) * MN) + i);
          v[0] = v[0] + q[0];
          v[1] = v[1] + q[1];
          v[2] = v[2] + q[2];
          v[3] = v[3] + q[3];
        }
        d[i] = v;
      }
    }
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_rowgemm(const RowGemmParams& P, int kind, bool bf16, int64_t grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (bf16) {
    switch (kind) {
      case kGemmFc1Fwd: rowgemm_bf16_kernel<bf::MNC, kEpiStoreAct, 256><<<grid, 256, 0, st>>>(P); break;
      case kGemmFc2Fwd: rowgemm_bf16_kernel<bf::MNC, kEpiStore, 256><<<grid, 256, 0, st>>>(P); break;
      case kGemmFc2Dgrad: rowgemm_bf16_kernel<bf::KC, kEpiDgrad2, 256><<<grid, 256, 0, st>>>(P); break;
      case kGemmFc1Dgrad:
        if (P.list_hdr == 2)
          rowgemm_bf16_kernel<bf::KC, kEpiStore, kRowTile2><<<grid, 256, 0, st>>>(P);
        else
          rowgemm_bf16_kernel<bf::KC, kEpiStore, 256><<<grid, 256, 0, st>>>(P);
        break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (kind) {
      case kGemmFc1Fwd: rowgemm_f32_kernel<true, kEpiStoreAct><<<grid, 256, 0, st>>>(P); break;
      case kGemmFc2Fwd: rowgemm_f32_kernel<true, kEpiStore><<<grid, 256, 0, st>>>(P); break;
      case kGemmFc2Dgrad: rowgemm_f32_kernel<false, kEpiDgrad2><<<grid, 256, 0, st>>>(P); break;
      case kGemmFc1Dgrad: rowgemm_f32_kernel<false, kEpiStore><<<grid, 256, 0, st>>>(P); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_wgrad(const WgradParams& P, int which, bool bf16, int64_t grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (bf16) return hipErrorInvalidValue;  // bf16 runs launch_wgrad_pair
  if (which == 1)
    wgrad_f32_kernel<true, false><<<grid, 256, 0, st>>>(P);
  else
    wgrad_f32_kernel<false, true><<<grid, 256, 0, st>>>(P);
  return hipGetLastError();
}

hipError_t launch_wgrad_pair(const WgradParams& P1, const WgradParams& P2, int ncu, int64_t grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  wgrad_pair_bf16_kernel<<<grid, 256, 0, st>>>(P1, P2, ncu);
  return hipGetLastError();
}

hipError_t launch_mx_rowgemm(const RowGemmParams& P, int kind, int64_t grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (kind == kGemmFc2Dgrad)
    mx_rowgemm_kernel<256, kEpiDgrad2><<<grid, 256, 0, st>>>(P);
  else if (kind == kGemmFc1Fwd)
    mx_rowgemm_kernel<256, kEpiStoreAct><<<grid, 256, 0, st>>>(P);
  else if (kind != kGemmFc1Dgrad && kind != kGemmFc2Fwd)
    return hipErrorInvalidValue;
  else if (P.list_hdr == 2)
    mx_rowgemm_kernel<kRowTile2, kEpiStore><<<grid, 256, 0, st>>>(P);
  else
    mx_rowgemm_kernel<256, kEpiStore><<<grid, 256, 0, st>>>(P);
  return hipGetLastError();
}

hipError_t launch_wgrad_prep(const WgradPrepParams& P, bool bf16, int64_t grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (bf16)
    wgrad_prep_kernel<uint16_t><<<grid, 256, 0, st>>>(P);
  else
    wgrad_prep_kernel<float><<<grid, 256, 0, st>>>(P);
  return hipGetLastError();
}

hipError_t launch_wgrad_reduce(const WgradPrepParams& P, int64_t grid, hipStream_t st) {
  wgrad_reduce_kernel<<<grid, 256, 0, st>>>(P);
  return hipGetLastError();
}

int gemm_tile_m(bool bf16) { return bf16 ? bf::BM : f32::BM; }
int gemm_tile_n(bool bf16) { return bf16 ? bf::BN : f32::BN; }

}  // namespace moedet
