// Internal kernel parameter blocks and host-side launchers of libmoedet.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moedet {

constexpr int kMaxExperts = 1024;     // router width handled by the routing kernels
constexpr int kMaxTopK = 64;          // one lane per selected expert
constexpr int kRouteChunk = 16;       // tokens per routing/permutation chunk (two per wave of a route workgroup)
constexpr int kMaxChunkRows = 4096;   // upper bound on the wgrad K chunk (rows)
constexpr int64_t kManyWgradTiles = 8192;  // weight-gradient tiles above which no expert is split

// Grid size (a multiple of the 8 XCDs) for an upper bound on work units.
inline int64_t grid_for_units(int64_t U_max) { return ((U_max + 7) / 8) * 8; }
// grid for map_unit_rounds
inline int64_t grid_for_unit_rounds(int64_t U_max) { return grid_for_units(U_max) + 8; }

enum { kEpiStore = 0, kEpiDgrad2 = 1, kEpiStoreAct = 2 };
enum { kGemmFc1Fwd = 0, kGemmFc2Fwd = 1, kGemmFc2Dgrad = 2, kGemmFc1Dgrad = 3 };

struct RowGemmParams {
  const int32_t* counts;
  const int32_t* offsets;
  int groups;
  int N, K;
  const void* a;
  int64_t lda;
  uint32_t a_bytes;       // extent of a when gathered by a_rows (buffer range check);
                          // unread otherwise: a tile's own rows are addressed from its first
  const int32_t* a_rows;  // A row r reads a[a_rows[r]] when set, a[r] otherwise
  const void* b;
  int64_t b_gstride;      // elements between consecutive experts' B
  int64_t ldb;
  uint32_t b_bytes;       // extent of one expert's B
  void* c;
  int64_t ldc;
  void* c2;               // second output (a = relu(h)^2, or p*relu(h)^2)
  int64_t ldc2;
  // fc2 dgrad epilogue
  const void* h;
  int64_t ldh;
  const float* row_prob;
  const int32_t* row_src;
  float* part;  // [rows_cap][n_tiles]
  int n_tiles;
  float* dprob;
  int atomic;
  int ncu;                // compute units of the device (work-unit rounds)
  const int32_t* sched;   // routing.sched
  int list_hdr;           // header word holding the row-tile count (0 or 2)
  int64_t list_at;        // int32 offset of the row-tile entries
  // Side job run by the workgroups after the GEMM tiles (fc1 dgrad, which
  // leaves compute units idle at small shapes): the fixed-order dprob
  // combine of part[] (n_tiles partials per row) for side_nslot flat slots.
  // Workgroups [gemm_grid, gemm_grid + side_units) run the side units, after
  // every GEMM workgroup in dispatch order, so the GEMM tiles keep their
  // XCD-aware placement.
  const int32_t* side_slot_row;
  int64_t side_nslot;
  int side_units;
  int64_t gemm_grid;
  uint64_t seed;
  // MXFP8 row GEMM: E8M0 scales, one byte per 32 k, [rows][K/32]
  const uint8_t* a_scales;
  const uint8_t* b_scales;
  int64_t b_sgstride;     // scale bytes between consecutive experts' B
};
constexpr int kMxMaxK = 2048;  // K bound of the MXFP8 row GEMM (its scales are staged in LDS)
// MXFP8 weight-gradient operands: each expert's rows padded to a multiple of
// kMxPad (two 32-row blocks, one 64-element step of the scaled MFMA)
constexpr int kMxPad = 64;

// MXFP8 weight gradients: dW1_g = X_g^T dH_g and dW2_g = A_g^T dY_g from
// operands quantised along the routed rows, stored slice-major (codes
// [rpad / 64][cols][64], scales [rpad / 64][cols][2]; expert g owns padded
// rows poff[g] .. poff[g+1]).
struct MxWgradParams {
  const int32_t* poff;    // el + 1 padded row offsets (routing.sched)
  int groups;             // local experts
  int D, F;
  int64_t rpad;           // padded rows (a multiple of 64)
  const uint8_t* x_codes; const uint8_t* x_scales;      // [D][rpad]
  const uint8_t* dh_codes; const uint8_t* dh_scales;    // [F][rpad]
  const uint8_t* act_codes; const uint8_t* act_scales;  // [F][rpad]
  const uint8_t* dy_codes; const uint8_t* dy_scales;    // [D][rpad]
  float* dw1;             // [groups][D][F]
  float* dw2;             // [groups][F][D]
  uint64_t seed;
};

// Rows the weight-gradient quantiser reads (moe_mxw_src of the C ABI).
enum { kMxwToken = 0, kMxwRow = 1, kMxwActP = 2 };
struct MxWgradQuantParams {
  const uint16_t* src;    // bf16: [tokens][cols] (token), [rows_cap][cols] (row, act_p: h)
  int kind;
  int64_t cols;
  int64_t rpad;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* poff;
  int el;
  const int32_t* row_tok;
  const float* row_prob;
  uint8_t* codes;         // [rpad / 64][cols][64]
  uint8_t* scales;        // [rpad / 64][cols][2]
  uint64_t seed;
};

constexpr int kSideSlots = 1024;  // flat slots per side unit

struct WgradParams {
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* row_tok;
  const int32_t* units;  // routing.sched: [1] = unit count; entries at `units_at`
  int64_t units_at;
  int64_t aux_at;        // routing.sched: {S, chunk, first slot, 0} per unit
  int32_t* tickets;      // [wslots][tiles] arrival counters of split tiles (zeroed by the prologue)
  const int32_t* sched;  // unit_start[G+1], slot_base[G+1]
  int groups;
  int M, N;
  // the operand gathered by token (x or dy) has an extent (a_bytes or
  // b_bytes, below 2 GiB); the routed-row one (dh or act_p) is addressed
  // from each chunk's first row and its extent field is unread
  const void* a;
  int64_t lda;
  uint32_t a_bytes;
  const void* b;
  int64_t ldb;
  uint32_t b_bytes;
  float* dw;
  float* slots;
  int kc;
  int atomic;
  uint64_t seed;
};

struct RouterParams {
  int64_t T;
  int k, E, D;
  const int32_t* topk_idx;
  const float* topk_prob;
  const float* dprob;
  const int32_t* offsets;
  const int32_t* counts;
  const int32_t* row_tok;
  const void* x;
  const void* wr;
  float* dlogits;
  float* dwr;
  void* dx;
  int phases;  // dwr row phases: 8 or 64
  int atomic;
  uint64_t seed;
};

// Prologue of moe_bwd_wgrad (one launch): act_p = p relu(h)^2 over the
// routed rows, the float32 path's split-K schedule (block 0, when sched is
// set), zeroed arrival tickets, and in atomic mode zeroed dW of every split
// expert.
struct WgradPrepParams {
  const int32_t* counts;
  const int32_t* offsets;
  int32_t* sched;        // float32 path: unit_start[G+1], slot_base[G+1]; else null
  int groups;
  int M, N;
  int kc;
  int atomic;
  float* dw1;
  float* dw2;
  const float* slots1;
  const float* slots2;
  const void* h;         // [rows_cap, N] saved pre-activation (N = F)
  const float* row_prob;
  void* act_p;           // [rows_cap, N] output
  int32_t* tickets;
  int64_t n_tickets;
};

struct RouteParams {
  const float* logits;
  int64_t T;
  int E, k, eb, el;
  int32_t* topk_idx;
  float* topk_prob;
  int32_t* hist;  // [nchunk][el]
  int32_t* counts;
  int32_t* offsets;
  int32_t* cursor;  // [el] (atomic mode)
  int32_t* row_src;
  int32_t* row_tok;
  float* row_prob;
  int32_t* slot_row;
  int nchunk;
  int atomic;
  uint64_t seed;
  // backward work list (routing.sched)
  int32_t* sched;
  int bm;            // row-tile height of the backward GEMMs
  int bm2;           // row-tile height of the second list (fc1 dgrad)
  int kc;            // weight-gradient K chunk (rows)
  int64_t mt_cap;    // capacity of the row-tile list
  int64_t list2_at;  // int32 offset of the second row-tile list
  int64_t aux_at;    // int32 offset of the weight-gradient unit side table
  int64_t pad_at;    // int32 offset of the padded row offsets
};

// routing.sched: [0] row tiles of bm rows, [1] weight-gradient units,
// [2] row tiles of bm2 rows, [3] 0; then mt_cap row-tile entries {expert,
// first row in the expert, first row overall, rows}, wu_cap weight-gradient
// unit entries {expert | split << 30, first row, rows, partial slot or -1},
// mt_cap2 row-tile entries of bm2 rows, and wu_cap unit side entries
// {S, chunk, first partial slot of the expert, 0}, four int32 each; then
// el + 1 padded row offsets: each expert's row count rounded up to a
// multiple of kMxPad, prefix-summed (the column ranges of the MXFP8
// weight-gradient operands).
constexpr int kSchedHeader = 4;
constexpr int kRowTile2 = 192;  // bf16 fc1 dgrad row tile: two waves of 96 rows

hipError_t launch_route(const RouteParams& P, hipStream_t st);
hipError_t launch_permute_scan(const RouteParams& P, hipStream_t st);
hipError_t launch_permute_scatter(const RouteParams& P, hipStream_t st);

hipError_t launch_rowgemm(const RowGemmParams& P, int kind, bool bf16, int64_t grid, hipStream_t st);
hipError_t launch_wgrad(const WgradParams& P, int which, bool bf16, int64_t grid, hipStream_t st);
hipError_t launch_wgrad_prep(const WgradPrepParams& P, bool bf16, int64_t grid, hipStream_t st);
hipError_t launch_wgrad_reduce(const WgradPrepParams& P, int64_t grid, hipStream_t st);
// bf16: both weight gradients (P1: dW1, P2: dW2) in one launch, schedule computed in-kernel
hipError_t launch_wgrad_pair(const WgradParams& P1, const WgradParams& P2, int ncu, int64_t grid, hipStream_t st);
int gemm_tile_m(bool bf16);
int gemm_tile_n(bool bf16);

// combine / dprob kernels
hipError_t launch_gather_combine(const void* rows, const int32_t* slot_row, const float* weights,
                                 int64_t T, int k, int D, void* out, bool bf16, uint64_t seed,
                                 hipStream_t st);
hipError_t launch_scatter_add(const void* rows, const int32_t* offsets, int el,
                              const int32_t* row_tok, const float* row_prob, int64_t rows_cap, int D,
                              float* out32, bool bf16, uint64_t seed, hipStream_t st);
hipError_t launch_cast(const float* in32, void* out, int64_t n, bool bf16, hipStream_t st);
hipError_t launch_zero(float* p, int64_t n, hipStream_t st);
hipError_t launch_router_bwd(const RouterParams& P, bool bf16, hipStream_t st);
hipError_t launch_router_fwd(const void* x, const void* wr, int64_t T, int E, int D, float* logits, bool bf16,
                             uint64_t seed, hipStream_t st);
// MXFP8 row GEMM: kind kGemmFc1Dgrad or kGemmFc2Fwd (bf16 rows of C; P.list_hdr
// 2 selects the 192-row tiles), kGemmFc2Dgrad (the fc2 dgrad epilogue) or
// kGemmFc1Fwd (h and relu(h)^2 rows); 256-row tiles unless stated.
hipError_t launch_mx_rowgemm(const RowGemmParams& P, int kind, int64_t grid, hipStream_t st);
hipError_t launch_mx_wgrad(const MxWgradParams& P, hipStream_t st);
hipError_t launch_mx_quantize_wgrad(const MxWgradQuantParams& P, hipStream_t st);
hipError_t launch_nvfp4_quantize(const void* in, bool bf16, int64_t rows, int64_t cols, uint8_t* codes,
                                 uint8_t* scales, float* global_scale, uint64_t seed, hipStream_t st);
hipError_t launch_mx_quantize(const void* in, bool bf16, int64_t rows, int64_t cols, uint8_t* codes,
                              uint8_t* scales, uint64_t seed, hipStream_t st);
hipError_t launch_mx_quantize_t(const void* in, bool bf16, int64_t groups, int64_t rows, int64_t cols,
                                uint8_t* codes, uint8_t* scales, uint64_t seed, hipStream_t st);
hipError_t launch_sgd(float* master, const float* grad, int64_t n, float lr, void* runtime, bool bf16,
                      hipStream_t st);
hipError_t launch_dprob_combine(const float* part, const int32_t* slot_row, int64_t nslots, int n_tiles,
                                float* dprob, uint64_t seed, hipStream_t st);

// fingerprint
hipError_t launch_mfma_rate(int64_t blocks, int64_t iters, float v, float* sink, hipStream_t st);
hipError_t launch_fingerprint(const void* data, int width, int64_t n, int64_t chunk,
                              const uint64_t* words, int nwords, uint64_t* chunk_hashes,
                              uint64_t* total, hipStream_t st);

}  // namespace moedet
