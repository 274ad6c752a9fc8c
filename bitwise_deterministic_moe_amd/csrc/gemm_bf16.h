// bf16 grouped-GEMM main loop for gfx950.
//
// Tile 256x256, K slice 32, 4 waves in a 2x2 grid, each wave 128x128 as 4x4
// blocks of v_mfma_f32_32x32x16_bf16 (accumulators in AGPRs).  Operands go
// from HBM straight into LDS with buffer_load_dwordx4 ... lds (no VGPR
// staging) through a ring of 4 or 5 slots, so two and a half (three and a
// half) K slices are in flight while one is consumed.  Rows outside the group / K range are given an offset
// past the buffer's num_records, for which the hardware writes zeros.
//
// LDS layouts (bf16 elements):
//  KC  operand contiguous along K in memory: tile [256 rows][32 k], rows of
//      64 bytes; the 16-byte chunk c of row r sits at c ^ ((r>>2)&3).
//  MNC operand contiguous along M/N: tile [32 k][256 mn], rows of 512 bytes;
//      chunk c of row k sits at c ^ 4*(k&7).
//  Both XOR patterns were chosen by measuring the LDS bank-conflict counter
//  on gfx950 for the exact fragment access patterns below (the LDS moves
//  256 bytes per clock; several patterns that look conflict-free under a
//  plain "16 lanes x 16 bytes per cycle" model are 2-way conflicted there).
//  The DMA writes are 1 KiB contiguous per instruction and conflict-free.
//  Fragments of MNC operands are read with
//      ds_read_b64_tr_b16: in a group of 16 lanes, lane i supplies the address
//      of 4 consecutive mn values of row k0 + i/4 (mn = n0 + 4*(i%4)) and
//      receives the 4 values of rows k0..k0+3 at column n0 + i.
// A fragment lane l always holds row/column (l % 32) of its 32-block and
// k = 16*kk + 8*(l/32) + 0..7 of the current slice, for both layouts.
#pragma once

#include "common.h"

#define LDS_AS __attribute__((address_space(3)))

namespace moedet {
namespace bf {

constexpr int BM = 256, BN = 256, BK = 32, NSTAGE = 4, NT = 256;
constexpr int OPER = BM * BK;                 // elements per operand per stage
constexpr int STAGE = 2 * OPER;               // A then B
constexpr int LDS_BYTES = NSTAGE * STAGE * 2; // 128 KiB
// Ring of NS slots: NS = 5 fills the 160 KiB of LDS of a gfx950 CU.
template <int NS>
constexpr int ring_bytes = NS * STAGE * 2;
constexpr int LOADS = 4;                      // 16-byte DMA loads per thread per operand per stage
constexpr uint32_t kOOB = 0x80000000u;        // offset beyond any num_records: reads zeros

enum { KC = 0, MNC = 1 };

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

typedef short v4i16 __attribute__((ext_vector_type(4)));

DEV int kc_swz(int r) { return (r >> 2) & 3; }
DEV int mnc_swz(int k) { return (k & 7) << 2; }
DEV int kc_off(int r, int c) { return r * 32 + ((c ^ kc_swz(r)) << 3); }
DEV int mnc_off(int k, int mn) { return k * 256 + (((mn >> 3) ^ mnc_swz(k)) << 3) + (mn & 7); }

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: base, stride 0, num_records = bytes, default format.
DEV i32x4_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return i32x4_t{(int)(uint32_t)a, (int)((a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// LDS byte address of a __shared__ object (a link-time constant).
template <class T>
DEV uint32_t lds_base(T* p) {
  return (uint32_t)(uintptr_t)(LDS_AS T*)p;
}

// One 16-byte-per-lane DMA load HBM -> LDS: lane i's data lands at
// lds + 16*i.  Issued through asm so that the compiler does not insert a
// full vmcnt wait before every later LDS read; the main loop counts the
// outstanding loads itself.  ``lds`` and ``soff`` are wave-uniform.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
DEV void dma16(i32x4_t rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(l), "v"(voff), "s"(rs), "s"(so)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most N of this thread's DMA loads are outstanding, then
// meet the other waves.  The asm keeps the compiler from moving LDS reads
// across.
template <int N>
DEV void wait_barrier() {
  static_assert(N == 0 || N == 8 || N == 12 || N == 16 || N == 20, "vmcnt");
  if constexpr (N == 20)
    asm volatile("s_waitcnt vmcnt(20)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 16)
    asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 12)
    asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 8)
    asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

DEV void block_barrier() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ------------------------------------------------------------- fragments
DEV bf16x8_t frag_kc(const uint16_t* s, int row, int kk, int lane) {
  return __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(s + kc_off(row, kk * 2 + (lane >> 5))));
}

DEV bf16x8_t frag_mnc(const uint16_t* s, int col_base, int kk, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int k = kk * 16 + 8 * (g >> 1) + (i >> 2);
  const int mn = col_base + 16 * (g & 1) + 4 * (i & 3);
  v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(s + mnc_off(k, mn)));
  v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(s + mnc_off(k + 4, mn)));
  u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
  return __builtin_bit_cast(bf16x8_t, u32x4_t{l2[0], l2[1], h2[0], h2[1]});
}

template <int L>
DEV bf16x8_t frag(const uint16_t* s, int blk_base, int kk, int lane) {
  if constexpr (L == KC)
    return frag_kc(s, blk_base + (lane & 31), kk, lane);
  else
    return frag_mnc(s, blk_base, kk, lane);
}

struct Frags {
  bf16x8_t a[4], b[4];
};

// Fragment read addresses of an MNC x MNC tile for the unrolled main loop:
// per lane, the LDS byte addresses of the 16 transpose reads of k-half 0 in
// slot 0 (blocks A0..A3 then B0..B3, each a read of rows k and k+4), and the
// same addresses + 64 KiB.  A read of slot sl, k-half kh is then one of
// them plus (sl % 2) * 32 KiB + kh * 8 KiB, an offset that fits the
// instruction's 16-bit field, so no address arithmetic runs per read (rows
// k + 16 share the swizzle of rows k).  The second set goes through an asm
// add so that the compiler keeps it as registers instead of rebuilding
// addresses past the offset field.
struct MncAddr {
  uint32_t s0[16], s1[16];
};

template <int WTM>
DEV void mnc_addr_init(MncAddr& m, uint32_t ring, int wm, int wn, int lane) {
  const int g4 = lane >> 4, i = lane & 15;
  const int k = 8 * (g4 >> 1) + (i >> 2);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int col = (b >= 4 ? wn * 128 : wm * WTM) + (b & 3) * 32 + 16 * (g4 & 1) + 4 * (i & 3);
    const uint32_t base = ring + (b >= 4 ? (uint32_t)OPER * 2u : 0u);
    m.s0[2 * b] = base + 2u * (uint32_t)mnc_off(k, col);
    m.s0[2 * b + 1] = base + 2u * (uint32_t)mnc_off(k + 4, col);
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) asm("v_add_u32 %0, 0x10000, %1" : "=v"(m.s1[j]) : "v"(m.s0[j]));
}

DEV bf16x8_t frag_mnc_at(const MncAddr& m, int b, int sl, int kh) {
  const uint32_t* set = sl >= 2 ? m.s1 : m.s0;
  const uint32_t off = (uint32_t)(sl & 1) * 32768u + (uint32_t)kh * 8192u;
  const LDS_AS char* plo = (const LDS_AS char*)(uintptr_t)set[2 * b];
  const LDS_AS char* phi = (const LDS_AS char*)(uintptr_t)set[2 * b + 1];
  v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(plo + off));
  v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4i16*)(phi + off));
  u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
  return __builtin_bit_cast(bf16x8_t, u32x4_t{l2[0], l2[1], h2[0], h2[1]});
}

// Fragment reads and MFMAs of a k-half in 8 groups.  Group g reads block
// A0 B0 B1 A1 B2 B3 A2 A3 [g] and issues MFMA pair g:
//   (A0;B0,B1) (A1;B0,B1) (A0;B2,B3) (A1;B2,B3) (A2;B0,B1) (A2;B2,B3) (A3;B0,B1) (A3;B2,B3)
// so the pair of group g only needs blocks read by groups 0..g+1 of the
// previous phase, never the reads issued last.
constexpr int kGrpA[8] = {0, -1, -1, 1, -1, -1, 2, 3};
constexpr int kGrpB[8] = {-1, 0, 1, -1, 2, 3, -1, -1};
constexpr int kGrpM[8] = {0, 1, 0, 1, 2, 2, 3, 3};
constexpr int kGrpN[8] = {0, 0, 2, 2, 0, 2, 0, 2};

// NMB: number of the wave's 32-row A blocks that hold rows (4 for a full
// tile).  A wave of a partial tile skips the reads and MFMAs of the blocks
// past the group end, which would only multiply zeros.
// WTM: rows of the wave tile (128, or 96 for a 192-row tile).
template <int AL, int BL, int NMB = 4, int WTM = 128>
DEV void load_frag(Frags& f, const uint16_t* st, int kk, int wm, int wn, int lane, int g) {
  if (kGrpA[g] >= 0) {
    if (kGrpA[g] < NMB) f.a[kGrpA[g]] = frag<AL>(st, wm * WTM + kGrpA[g] * 32, kk, lane);
  } else {
    f.b[kGrpB[g]] = frag<BL>(st + OPER, wn * 128 + kGrpB[g] * 32, kk, lane);
  }
}

// FIRST: the tile's first k-half, whose MFMAs take a zero accumulator input
// (the same +0.0 the accumulators would hold), so no zeroing of the 256
// accumulator registers has to run after slice 0 has landed.
template <int NMB = 4, bool FIRST = false>
DEV void mma2(const Frags& f, f32x16_t (&acc)[4][4], int g) {
  const int mb = kGrpM[g], nb = kGrpN[g];
  if (mb >= NMB) return;
  const f32x16_t zero = {};
  acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[nb], f.a[mb], FIRST ? zero : acc[mb][nb], 0, 0, 0);
  acc[mb][nb + 1] =
      __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[nb + 1], f.a[mb], FIRST ? zero : acc[mb][nb + 1], 0, 0, 0);
}

template <int NMB>
DEV void load_frag_at(Frags& f, const MncAddr& m, int sl, int kh, int g) {
  if (kGrpA[g] >= 0) {
    if (kGrpA[g] < NMB) f.a[kGrpA[g]] = frag_mnc_at(m, kGrpA[g], sl, kh);
  } else {
    f.b[kGrpB[g]] = frag_mnc_at(m, 4 + kGrpB[g], sl, kh);
  }
}

DEV void mma16(const Frags& f, f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[nb], f.a[mb], acc[mb][nb], 0, 0, 0);
}

// ---------------------------------------------------------------- loaders
// Per-thread description of one operand's DMA loads.  Wave w issues the
// wave-loads j = 4w + i (i = 0..3); each wave-load fills 1 KiB of LDS.
//  KC : wave-load j covers tile rows 16j..16j+15; lane L loads row
//       16j + L/4, logical chunk (L%4) ^ ((row>>2)&3) at K offset k0.
//  MNC: wave-load j covers k rows 2j, 2j+1; lane L loads k row 2j + L/32,
//       logical chunk (L%32) ^ 4*(k&7).
struct KcOperand {
  i32x4_t rs;
  uint32_t voff[LOADS];  // row offset + chunk, bytes (kOOB for masked rows)
  // rowoff(r) -> byte offset of tile row r (K start of the GEMM) or kOOB
  template <class RowOff>
  DEV void init(const void* base, uint32_t bytes, int wave, int lane, RowOff rowoff) {
    rs = make_rsrc(base, bytes);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int j = wave * LOADS + i;
      const int r = 16 * j + (lane >> 2);
      const int c = (lane & 3) ^ kc_swz(r);
      const uint32_t ro = rowoff(r);
      voff[i] = ro == kOOB ? kOOB : ro + (uint32_t)c * 16u;
    }
  }
  // Load i of this operand for the slice at K offset k0; lds: byte address
  // of the operand's tile in the slot (uniform); live == false issues the
  // load past the buffer end.
  DEV void issue1(uint32_t lds, int wave, int k0, bool live, int i) const {
    issue1_bytes(lds, wave, (uint32_t)k0 * 2u, live, i);
  }
  // The same with the slice's byte offset from the tile's rows given directly.
  DEV void issue1_bytes(uint32_t lds, int wave, uint32_t soff, bool live, int i) const {
    dma16(rs, lds + (wave * LOADS + i) * 1024, live ? voff[i] : kOOB, live ? soff : 0u);
  }
};

struct MncOperand {
  i32x4_t rs;
  uint32_t mnoff[LOADS];  // byte offset of this lane's 8 mn values inside a k row
  DEV void init(const void* base, uint32_t bytes, int wave, int lane, int mn0) {
    rs = make_rsrc(base, bytes);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int j = wave * LOADS + i;
      const int k = 2 * j + (lane >> 5);
      const int c = (lane & 31) ^ mnc_swz(k);
      mnoff[i] = (uint32_t)(mn0 + 8 * c) * 2u;
    }
  }
  // krowoff(k) -> byte offset of k row (k relative to the stage start) or kOOB
  // k row handled by this lane in load i
  DEV static int krow(int wave, int lane, int i) { return 2 * (wave * LOADS + i) + (lane >> 5); }
  // Load i; ro: byte offset of k row krow(i) of the slice, or kOOB.  Then
  // ro + mnoff[i] is at or past 2^31: past num_records of any buffer under
  // 2 GiB, which reads zeros; in a larger weight buffer it reads in-range
  // data into a slot that is never read (slices past the last one).
  DEV void issue1(uint32_t lds, int wave, uint32_t ro, int i) const {
    dma16(rs, lds + (wave * LOADS + i) * 1024, ro + mnoff[i], 0u);
  }
};

// Pipelined main loop over nsteps K slices through a ring of NS LDS slots
// (slice s in slot s % NS).  issue(s, lds, i) issues DMA load i (0..3 of A,
// 4..7 of B) of slice s into the slot at LDS byte address lds; loads of a
// slice are requested in order i = 0..7 and slices in increasing order.  For
// s >= nsteps every load must carry an offset past the buffer end (no
// memory traffic; zeros land in a slot that is never read again), which
// keeps the outstanding-load count the same in every step.  NS - 2 slices
// and a half are in flight while one is consumed, which covers the HBM
// latency of a loaded device with NS = 5.
//
// A wave issues instructions in order, and a DMA load occupies the
// per-CU address path for about 16 clocks, so loads are spread evenly over
// the step (one per four MFMAs) instead of in a burst, and each LDS
// fragment read sits next to the MFMAs it overlaps (scheduling barriers
// pin the order):
//  phase 1 of step s: fragments of slice s / k-half 1 are read and loads
//    4..7 of slice s+NS-2 issued, while the MFMAs of k-half 0 run;
//  wait for this wave's loads of slice s+1, meet the other waves (every wave
//    is then done with slice s-1, whose slot takes slice s+NS-1);
//  phase 2: fragments of slice s+1 / k-half 0 are read and loads 0..3 of
//    slice s+NS-1 issued, while the MFMAs of k-half 1 run.
// UNR: the steady-state loop is unrolled NS times, so that every slot
// index, and with it every LDS address offset, is a compile-time constant
// (the fragment reads then take the slot in their immediate offset instead of
// an add per read); the up to NS - 1 steps left after the unrolled rounds
// start at slot 1 as well.
template <int AL, int BL, int NMB = 4, int NS = NSTAGE, int WTM = 128, bool UNR = false, class Issue>
DEV void mainloop(const uint16_t* lds, uint32_t ring, int nsteps, Issue issue, f32x16_t (&acc)[4][4], int wm,
                  int wn, int lane) {
  static_assert(NS == 4 || NS == 5, "ring slots");
  if (nsteps <= 0) return;
  auto slot = [&](int s) { return lds + (s % NS) * STAGE; };
  auto slot_addr = [&](int s) { return ring + (uint32_t)(s % NS) * (STAGE * 2); };
#pragma unroll
  for (int s = 0; s < NS - 2; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) issue(s, slot_addr(s), i);
#pragma unroll
  for (int i = 0; i < 4; ++i) issue(NS - 2, slot_addr(NS - 2), i);
  wait_barrier<8 * (NS - 3) + 4>();  // slice 0 landed
  Frags f0, f1;
#pragma unroll
  for (int g = 0; g < 8; ++g) load_frag<AL, BL, NMB, WTM>(f0, lds, 0, wm, wn, lane, g);
  if (nsteps == 1) {
#pragma unroll
    for (int g = 0; g < 8; ++g) load_frag<AL, BL, NMB, WTM>(f1, lds, 1, wm, wn, lane, g);
#pragma unroll
    for (int g = 0; g < 8; ++g) mma2<NMB, true>(f0, acc, g);
#pragma unroll
    for (int g = 0; g < 8; ++g) mma2<NMB>(f1, acc, g);
    block_barrier();
    return;
  }
  static_assert(!UNR || (AL == MNC && BL == MNC && NS == 4), "unrolled loop: MNC x MNC tiles, 4 slots");
  MncAddr ma;
  if constexpr (UNR) mnc_addr_init<WTM>(ma, ring, wm, wn, lane);
  // phase 1 of step s, whose slice sits in slot sl = s % NS (the MFMAs of
  // slice s / k-half 0)
  auto phase1 = [&](int s, auto first, int sl) __attribute__((always_inline)) {
    const uint16_t* cur = lds + sl * STAGE;
    const int si = sl >= 2 ? sl - 2 : sl + NS - 2;  // slot of slice s + NS - 2
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if (g & 1) issue(s + NS - 2, ring + (uint32_t)si * (STAGE * 2), 4 + (g >> 1));
      if constexpr (UNR)
        load_frag_at<NMB>(f1, ma, sl, 1, g);
      else
        load_frag<AL, BL, NMB, WTM>(f1, cur, 1, wm, wn, lane, g);
      __builtin_amdgcn_sched_barrier(0);
      mma2<NMB, decltype(first)::value>(f0, acc, g);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // wait, then phase 2 of step s (the MFMAs of slice s / k-half 1)
  auto phase2 = [&](int s, int sl) __attribute__((always_inline)) {
    const uint16_t* nxt = lds + (sl + 1 == NS ? 0 : sl + 1) * STAGE;
    const int si = sl >= 1 ? sl - 1 : NS - 1;  // slot of slice s + NS - 1
    wait_barrier<8 * (NS - 3)>();  // slice s+1 landed; slot of slice s-1 free
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if (g & 1) issue(s + NS - 1, ring + (uint32_t)si * (STAGE * 2), g >> 1);
      if constexpr (UNR)
        load_frag_at<NMB>(f0, ma, sl + 1 == NS ? 0 : sl + 1, 0, g);
      else
        load_frag<AL, BL, NMB, WTM>(f0, nxt, 0, wm, wn, lane, g);
      __builtin_amdgcn_sched_barrier(0);
      mma2<NMB>(f1, acc, g);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  phase1(0, BoolC<true>{}, 0);
  phase2(0, 0);
  if constexpr (UNR) {
    int s = 1;
#pragma unroll 1
    for (; s + NS <= nsteps - 1; s += NS) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        phase1(s + j, BoolC<false>{}, (1 + j) % NS);
        phase2(s + j, (1 + j) % NS);
      }
    }
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) {
      if (s + j < nsteps - 1) {
        phase1(s + j, BoolC<false>{}, (1 + j) % NS);
        phase2(s + j, (1 + j) % NS);
      }
    }
  } else {
#pragma unroll 1
    for (int s = 1; s < nsteps - 1; ++s) {
      phase1(s, BoolC<false>{}, s % NS);
      phase2(s, s % NS);
    }
  }
#pragma unroll
  for (int g = 0; g < 8; ++g) load_frag<AL, BL, NMB, WTM>(f1, slot(nsteps - 1), 1, wm, wn, lane, g);
#pragma unroll
  for (int g = 0; g < 8; ++g) mma2<NMB>(f0, acc, g);
#pragma unroll
  for (int g = 0; g < 8; ++g) mma2<NMB>(f1, acc, g);
  block_barrier();
}

}  // namespace bf
}  // namespace moedet
