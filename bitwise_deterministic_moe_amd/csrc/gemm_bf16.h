// bf16 grouped-GEMM main loop for gfx950.
//
// Tile 256x256, K slice 32, 4 waves in a 2x2 grid, each wave 128x128 as 4x4
// blocks of v_mfma_f32_32x32x16_bf16 (accumulators in AGPRs).  Operands go
// from HBM straight into LDS with buffer_load_dwordx4 ... lds (no VGPR
// staging) through a 4-stage ring, so three K slices are in flight while
// one is consumed.  Rows outside the group / K range are given an offset
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
constexpr int LOADS = 4;                      // 16-byte DMA loads per thread per operand per stage
constexpr uint32_t kOOB = 0x80000000u;        // offset beyond any num_records: reads zeros

enum { KC = 0, MNC = 1 };

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

DEV uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(const LDS_AS void*)p; }

// One 16-byte-per-lane DMA load HBM -> LDS: lane i's data lands at
// lds + 16*i.  Issued through asm so that the compiler does not insert a
// full vmcnt wait before every later LDS read; the main loop counts the
// outstanding loads itself.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
DEV void dma16(i32x4_t rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);  // wave-uniform by construction
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
DEV void wait_barrier(int n_outstanding) {
  if (n_outstanding >= 16)
    asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  else if (n_outstanding >= 8)
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

template <int AL, int BL>
DEV void load_frags(Frags& f, const uint16_t* st, int kk, int wm, int wn, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = frag<AL>(st, wm * 128 + i * 32, kk, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) f.b[i] = frag<BL>(st + OPER, wn * 128 + i * 32, kk, lane);
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
  DEV void issue(uint16_t* stage_base, int wave, int k0) const {
#pragma unroll
    for (int i = 0; i < LOADS; ++i)
      dma16(rs, lds_addr(stage_base + (wave * LOADS + i) * 512), voff[i], (uint32_t)k0 * 2u);
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
  template <class KRowOff>
  DEV void issue(uint16_t* stage_base, int wave, int lane, KRowOff krowoff) const {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int k = 2 * (wave * LOADS + i) + (lane >> 5);
      const uint32_t ro = krowoff(k);
      dma16(rs, lds_addr(stage_base + (wave * LOADS + i) * 512), ro == kOOB ? kOOB : ro + mnoff[i], 0u);
    }
  }
};

// Pipelined main loop over nsteps K slices.  issue(s, stage_ptr) must issue
// exactly 2*LOADS DMA loads per thread (A into stage_ptr, B into
// stage_ptr + OPER).
//
// Iteration s: fragments of slice s / k-half 1 are read while the MFMAs of
// k-half 0 run; then the wave waits for its DMA loads of slice s+1 and meets
// the others at the barrier (which also proves every wave is done with
// slice s-1, whose ring slot is refilled with slice s+3); then slice s+1 /
// k-half 0 fragments are read while the MFMAs of k-half 1 run.  DMA loads
// are therefore issued two iterations before they are needed.
template <int AL, int BL, class Issue>
DEV void mainloop(uint16_t* lds, int nsteps, Issue issue, f32x16_t (&acc)[4][4], int wm, int wn, int lane) {
  if (nsteps <= 0) return;
  const int pre = nsteps < NSTAGE - 1 ? nsteps : NSTAGE - 1;
  for (int s = 0; s < pre; ++s) issue(s, lds + s * STAGE);
  wait_barrier(2 * LOADS * (pre - 1));
  Frags f0, f1;
  load_frags<AL, BL>(f0, lds, 0, wm, wn, lane);
  for (int s = 0; s < nsteps; ++s) {
    const uint16_t* st = lds + (s % NSTAGE) * STAGE;
    load_frags<AL, BL>(f1, st, 1, wm, wn, lane);
    mma16(f0, acc);
    if (s + 1 < nsteps) {
      // outstanding after slice s+1: slice s+2 if it was issued
      wait_barrier(s + 2 < nsteps ? 2 * LOADS : 0);
      if (s + NSTAGE - 1 < nsteps) issue(s + NSTAGE - 1, lds + ((s + NSTAGE - 1) % NSTAGE) * STAGE);
      load_frags<AL, BL>(f0, lds + ((s + 1) % NSTAGE) * STAGE, 0, wm, wn, lane);
    }
    mma16(f1, acc);
  }
  block_barrier();
}

}  // namespace bf
}  // namespace moedet
