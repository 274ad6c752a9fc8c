/*
 * moedet.h -- bitwise-deterministic MoE expert layer for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libmoedet.so.  Every compute entry point takes a mode:
 *   MOE_DETERMINISTIC  every reduction runs in an order fixed by indices and
 *                      shapes only, so the output bits are a pure function of
 *                      the input bits, the problem description, the library
 *                      build and the GPU model;
 *   MOE_ATOMIC         the same kernels, but the reduction sites add with
 *                      floating-point atomics in arrival order (the fault the
 *                      pages describe), for comparison and as a negative
 *                      control.
 *
 * Sources (the pages):
 *   - "Trillion-Parameter Pretraining Goes Bitwise-Deterministic" (English
 *     digest), section "Interpretation": in the grouped-GEMM epilogue several
 *     N-tiles added into the same dprob[token] address, so the result depended
 *     on their arrival order; the fix gives every N-tile a private output slot
 *     and combines the slots in a fixed order once all writers have finished.
 *     The same section states the general rule (fix the reduction order, keep
 *     a full-precision source of truth).
 *   - The French article, section "Optimisation pour le Nemotron à mille
 *     milliards de paramètres": private output slots for the grouped-GEMM
 *     writers and a fixed reduction order that keeps the parallelism.
 *   - The French article, section "Méthodologie de débogage du
 *     non-déterminisme": GPU tensor fingerprints recording shape, dtype and
 *     element count, chunk-wise for order-sensitive data (routing maps, MoE
 *     dispatch outputs).
 *   The same fixed-order rule is applied here to the split-K expert weight
 *   gradient and to the top-k unpermute/combine.
 *
 * Conventions (all calls):
 *   - Tensor arguments are DEVICE pointers to row-major contiguous arrays,
 *     allocated and owned by the caller.  The library never allocates or
 *     frees memory and keeps no state between calls.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = default
 *     stream).  Calls return after enqueue, with no host synchronisation and
 *     no device-to-host copies.
 *   - Arguments are validated before anything is enqueued: a status other
 *     than MOE_OK (except MOE_ERR_HIP) means no work was enqueued.
 *     MOE_ERR_HIP reports a launch failure (hipGetLastError).
 *   - Inputs are read-only.  Every element of every output is written on
 *     every call, in both modes; outputs need no pre-zeroing.  Row-layout
 *     outputs ([rows_cap, .]) are written for rows < R only, where
 *     R = routing.offsets[num_local] (a device value).
 *   - Workspace contents are undefined on entry and on exit.  Size it with
 *     moe_workspace_size; it must be 256-byte aligned.
 *   - Calls that share a workspace or outputs must be ordered on one stream.
 *   - Storage dtype (problem.dtype) applies to x, W1, W2, dy, h, y, dh, dx
 *     and the row-layout outputs.  Routing probabilities, dprob and dW are
 *     always float32; accumulation is float32.
 *   - Non-finite logits give undefined routing.
 */
#ifndef MOEDET_H
#define MOEDET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,      /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,     /* invalid sizes, alignment or expert range */
  MOE_ERR_DTYPE = 3,     /* unsupported dtype */
  MOE_ERR_WORKSPACE = 4, /* workspace too small or misaligned */
  MOE_ERR_MODE = 5,      /* unknown mode or combine flag */
  MOE_ERR_HIP = 6        /* a HIP launch or event call failed */
} moe_status;

typedef enum moe_dtype {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_I32 = 2,
  MOE_U8 = 3,
  MOE_I64 = 4,
  MOE_F64 = 5
} moe_dtype;

typedef enum moe_mode { MOE_DETERMINISTIC = 0, MOE_ATOMIC = 1 } moe_mode;

/* Layer description.
 *   tokens        T >= 0 tokens of this call
 *   d_model       D, the expert input/output width (the LatentMoE latent)
 *   d_ffn         F, the expert hidden width; expert MLP o = relu(x W1)^2 W2,
 *                 no bias, W1 [D,F], W2 [F,D]
 *   num_experts   E, router width (1..1024)
 *   top_k         k, experts per token (1..min(E,64))
 *   expert_begin, num_local
 *                 the experts held here: [expert_begin, expert_begin+num_local)
 *   dtype         MOE_F32 (D, F multiples of 64) or MOE_BF16 (multiples of 256);
 *                 every [T,D] array below 2 GiB (T < 512K tokens at a bf16
 *                 D of 2048) and every [rows_cap,max(D,F)] array below 32 GiB
 *   combine       1: full layer, outputs in token layout ([T,D]; requires
 *                 num_local == num_experts);
 *                 0: expert shard, outputs in row layout ([rows_cap,D]) as an
 *                 expert-parallel rank would send them back
 *   debug_shuffle_seed
 *                 0 = off.  Otherwise every kernel permutes the order in which
 *                 its workgroups take work and delays some of them; in
 *                 MOE_DETERMINISTIC mode the results do not change.  Testing only.
 *   stage_events, n_stage_events
 *                 optional timing hook: NULL/0 = off.  Otherwise an array of
 *                 n_stage_events hipEvent_t handles owned by the caller; the
 *                 library records event i just before the i-th kernel of the
 *                 call and one more after its last kernel (events beyond
 *                 n_stage_events are skipped).  moe_stage_names lists the
 *                 kernels. */
typedef struct moe_problem {
  int64_t tokens;
  int32_t d_model;
  int32_t d_ffn;
  int32_t num_experts;
  int32_t top_k;
  int32_t expert_begin;
  int32_t num_local;
  int32_t dtype;
  int32_t combine;
  uint64_t debug_shuffle_seed;
  void* const* stage_events;
  int32_t n_stage_events;
} moe_problem;

/* Routing state: written by moe_fwd, read by the backward calls.
 * Flat slot index i = t*k + j.  rows_cap = T*min(k, num_local).
 *   topk_idx  [T,k]  int32   slot j holds the j-th largest logit's expert;
 *                            equal logits go to the lower expert index and
 *                            -0.0 equals +0.0
 *   topk_prob [T,k]  float   softmax over the k selected logits
 *   counts    [El]   int32   routed rows per local expert
 *   offsets   [El+1] int32   exclusive prefix of counts; offsets[El] = R
 *   row_src   [rows_cap] int32  row -> flat slot i; rows are grouped by local
 *                            expert and, in MOE_DETERMINISTIC mode, increasing
 *                            in i inside each expert (stable).  MOE_ATOMIC mode
 *                            claims rows with atomics, so the order inside an
 *                            expert is not fixed.
 *   row_tok   [rows_cap] int32  row -> token (= row_src / k)
 *   row_prob  [rows_cap] float  row -> topk_prob of its slot
 *   slot_row  [T*k]  int32   flat slot -> row, -1 when its expert is not local
 *   sched     [moe_sched_elems] int32  work list of the backward GEMMs, derived
 *                            from counts only (same in both modes): the row
 *                            tiles of the expert GEMMs, longest first, and the
 *                            (expert, K chunk) units of the weight gradients.
 *                            Its contents are private to the library. */
typedef struct moe_routing {
  int32_t* topk_idx;
  float* topk_prob;
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_src;
  int32_t* row_tok;
  float* row_prob;
  int32_t* slot_row;
  int32_t* sched;
} moe_routing;

/* ABI version (MOE_ABI_VERSION of the build). */
int moe_abi_version(void);

/* Hash of the sources the library was built from (16 hex digits of
 * SHA-256 over the csrc files and this header, as computed by the build
 * script), or "unknown" for a build that did not supply it.  Static string,
 * owned by the library. */
const char* moe_source_hash(void);

/* Static description of a status code. */
const char* moe_status_string(moe_status s);

/* rows_cap = tokens * min(top_k, num_local): leading size of row-layout buffers. */
moe_status moe_rows_cap(const moe_problem* p, int64_t* rows_cap);

/* Number of int32 elements of routing.sched for problem p (from shapes only). */
moe_status moe_sched_elems(const moe_problem* p, int64_t* elems);

/* Workspace bytes needed by each call for problem p in `mode` (upper bounds
 * from shapes only; no routing is read and nothing is enqueued).  The pages
 * describe no interface; the regions are this library's: routing histograms
 * and activation rows (fwd); the per-(row, N-tile) dprob partials, which are
 * the private output slots of the fix the English digest describes
 * ("Interpretation"), and the dx rows (dgrad); the split-K partial slots,
 * their arrival tickets and act_p = p relu(h)^2 (wgrad).  Any of the output
 * pointers may be NULL.  Errors: those of the problem's validation
 * (MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_MODE). */
moe_status moe_workspace_size(const moe_problem* p, moe_mode mode, size_t* fwd_bytes,
                              size_t* dgrad_bytes, size_t* wgrad_bytes);

/* Names of the kernels a call enqueues, in order, comma-separated, for the
 * stage_events hook.  call: 0 = moe_fwd, 1 = moe_bwd_dgrad_dprob,
 * 2 = moe_bwd_wgrad, 3 = moe_route.  Returns NULL for an invalid call or
 * problem. */
const char* moe_stage_names(const moe_problem* p, moe_mode mode, int call);

/* Forward: routing, stable permute, expert MLP and (combine=1) weighted
 * combine.  It produces the routing state and the saved activation that the
 * backward calls read.  Sources: the expert shapes follow the LatentMoE
 * description of the Nemotron 3 Ultra notes (section of concepts: a
 * 2048-wide latent, 512 experts, 22 selected); the combine is a gather over
 * the k slots in a fixed order, the reduction-order rule of the English
 * digest ("Interpretation") applied to the top-k combine.  The router's
 * tie-break, the softmax over the selected logits and the ReLU^2 expert MLP
 * are this library's readings (the pages state none of them).
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_MODE,
 * MOE_ERR_WORKSPACE before anything is enqueued; MOE_ERR_HIP for a launch
 * failure.
 *   logits     [T,E] float32
 *   x          [T,D] dtype
 *   w1         [El,D,F] dtype (local experts in order)
 *   w2         [El,F,D] dtype
 *   routing    its arrays are outputs (see moe_routing)
 *   h          [rows_cap,F] dtype  output: pre-activation h = x W1 per row,
 *              saved for the backward
 *   y_or_rows  combine=1: [T,D] y_t = sum_j p_tj o_(t,j), slots j ascending,
 *              float32 accumulation, rounded once;
 *              combine=0: [rows_cap,D] per-row expert outputs o
 *   ws         workspace of at least moe_workspace_size(...).fwd_bytes */
moe_status moe_fwd(const moe_problem* p, const float* logits, const void* x, const void* w1,
                   const void* w2, const moe_routing* routing, void* h, void* y_or_rows,
                   void* ws, size_t ws_bytes, moe_mode mode, void* stream);

/* The routing stage of moe_fwd alone (its first three kernels): top-k
 * selection with probabilities renormalised over the chosen experts, the
 * stable permutation of the (token, slot) pairs by local expert and the
 * backward work list, written to `routing` exactly as moe_fwd writes them
 * (same arguments, same workspace: the forward one of moe_workspace_size).
 * For callers that run the expert GEMMs through another path (the MXFP8
 * forward).  Errors: MOE_ERR_MODE, MOE_ERR_NULL, MOE_ERR_WORKSPACE and the
 * problem's validation before anything is enqueued; MOE_ERR_HIP for a
 * launch failure. */
moe_status moe_route(const moe_problem* p, const float* logits, const moe_routing* routing, void* ws,
                     size_t ws_bytes, moe_mode mode, void* stream);

/* Backward, data path: fc2 dgrad with the dprob epilogue, fc1 dgrad and the
 * dx combine.  This is the site of the fault and the fix in the English
 * digest ("Interpretation"): in the grouped-GEMM epilogue several N-tiles
 * added into the same dprob[token] address in arrival order; here every
 * N-tile writes a private float32 slot and the slots are combined in a fixed
 * order once all writers have finished (also the French article,
 * "Optimisation pour le Nemotron à mille milliards de paramètres": private
 * output slots for the grouped-GEMM writers).  The dx combine gathers the k
 * slots in a fixed order instead of scatter-adding.
 *   dy         [T,D] dtype upstream gradient of y (token layout also for the
 *              shard: row r reads dy[row_tok[r]])
 *   w1, w2     [El,D,F], [El,F,D] dtype, as given to moe_fwd
 *   h          [rows_cap,F] saved pre-activation from moe_fwd
 *   dx_or_rows combine=1: [T,D] dx_t = sum_j dx_(t,j), slots ascending;
 *              combine=0: [rows_cap,D] per-row dx
 *   dprob      [T,k] float32 dL/dp_tj = <dy_t, o_(t,j)>; 0 for slots whose
 *              expert is not local.  MOE_DETERMINISTIC: every N-tile of the
 *              fc2 dgrad writes a private float32 partial and a separate pass
 *              adds the partials in N-tile order.  MOE_ATOMIC: each N-tile
 *              adds its partial atomically.
 *   dh         [rows_cap,F] dtype output, p * (dy W2^T) * 2 relu(h); input of
 *              moe_bwd_wgrad
 *   ws         workspace of at least moe_workspace_size(...).dgrad_bytes
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_MODE,
 * MOE_ERR_WORKSPACE before anything is enqueued; MOE_ERR_HIP for a launch
 * failure. */
moe_status moe_bwd_dgrad_dprob(const moe_problem* p, const moe_routing* routing, const void* dy,
                               const void* w1, const void* w2, const void* h, void* dx_or_rows,
                               float* dprob, void* dh, void* ws, size_t ws_bytes, moe_mode mode,
                               void* stream);

/* Bytes of the device array that holds the workspace of
 * moe_bwd_dgrad_dprob_noalloc (one copy per GPU the library runs on). */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* moe_bwd_dgrad_dprob for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels, with the dgrad workspace taken from a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES per GPU (its device address is looked up once per
 * GPU, on the first call there) instead of a caller buffer.  The call
 * allocates and frees nothing.  Arguments and outputs are those of
 * moe_bwd_dgrad_dprob without ws / ws_bytes; the outputs are bit-identical
 * to moe_bwd_dgrad_dprob's in MOE_DETERMINISTIC mode.
 * Limit: the problem's dgrad workspace (moe_workspace_size(...).dgrad_bytes
 * for `mode`) must fit in MOE_NOALLOC_SCRATCH_BYTES, else MOE_ERR_WORKSPACE
 * is returned before anything is enqueued (for example the 4096-token,
 * 1024-wide, 8-expert top-2 layer needs 17 MB in MOE_DETERMINISTIC mode; a
 * 512-expert top-22 layer of 4096 tokens at width 2048 needs 372 MB and is
 * rejected).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other threads) race on it and must be serialised by the
 * caller.  The array keeps the last call's contents; nothing in it needs to
 * start at zero (what must be zeroed, the call zeroes itself).
 * Errors: those of moe_bwd_dgrad_dprob, plus MOE_ERR_WORKSPACE for a problem
 * beyond the limit and MOE_ERR_HIP if the array's address cannot be found. */
moe_status moe_bwd_dgrad_dprob_noalloc(const moe_problem* p, const moe_routing* routing, const void* dy,
                                       const void* w1, const void* w2, const void* h, void* dx_or_rows,
                                       float* dprob, void* dh, moe_mode mode, void* stream);

/* Backward, weight gradients (float32 outputs, exact zeros for experts
 * without rows):
 *   dw1 [El,D,F] = sum over the expert's rows of x_row^T dh_row
 *   dw2 [El,F,D] = sum over the expert's rows of act_p_row^T dy_row,
 *                  act_p = p * relu(h)^2, rebuilt from h into the workspace
 *                  by the call's first kernel
 * The pages name the weight-gradient path as one of the deterministic
 * paths that were optimised (English digest, "Interpretation"; French
 * article, "Optimisation pour le Nemotron à mille milliards de
 * paramètres"), and their rule -- a fixed reduction order -- is applied here
 * to the split-K sum.  An expert with many rows is split along its rows into
 * chunks whose size is a function of the problem shapes only.
 * MOE_DETERMINISTIC: chunk 0 stores its partial into dW, the other chunks
 * into workspace slots, and the chunk that finishes last (an integer ticket
 * per tile) adds them in chunk order, ((p0 + p1) + p2) + ...; which chunk
 * does the adding does not change the bits.  MOE_ATOMIC: the chunks are
 * added atomically into a zeroed dW.
 *   x, dy      [T,D] dtype (the layer input and the upstream gradient)
 *   h          [rows_cap,F] saved pre-activation from moe_fwd
 *   dh         [rows_cap,F] from moe_bwd_dgrad_dprob
 *   ws         workspace of at least moe_workspace_size(...).wgrad_bytes
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_MODE,
 * MOE_ERR_WORKSPACE before anything is enqueued; MOE_ERR_HIP for a launch
 * failure. */
moe_status moe_bwd_wgrad(const moe_problem* p, const moe_routing* routing, const void* x,
                         const void* dy, const void* h, const void* dh, float* dw1, float* dw2,
                         void* ws, size_t ws_bytes, moe_mode mode, void* stream);

/* Chunk-wise tensor fingerprint (integer arithmetic; bit-exact).
 *   data          device pointer to numel = prod(shape) elements of `dtype`
 *   shape         HOST array of ndim (0..8) sizes >= 0
 *   chunk_elems   C > 0 elements per chunk
 *   chunk_hashes  DEVICE uint64[ceil(numel/C)] output
 *   total         DEVICE uint64[1] output
 * Definition (mix64 = SplitMix64 finalizer, GAMMA = 0x9E3779B97F4A7C15,
 * arithmetic mod 2^64):
 *   v_i = mix64(bits_i ^ (i * GAMMA)), bits zero-extended element bits
 *   H_c = mix64((sum of v_i over chunk c) ^ c)
 *   total: h = GAMMA; for w in [dtype, ndim, shape..., numel, C, H_0, ...]:
 *          h = mix64(h ^ w) */
moe_status moe_fingerprint(const void* data, moe_dtype dtype, int ndim, const int64_t* shape,
                           int64_t chunk_elems, uint64_t* chunk_hashes, uint64_t* total,
                           void* stream);

/* Router backward, the step upstream of dprob ("Trillion-Parameter
 * Pretraining Goes Bitwise-Deterministic", section "Interpretation": the
 * grouped-GEMM epilogue produces dprob per token and selected expert; the
 * router consumes it).  Router: logits[t,e] = <x_t, wr_e>, the k largest
 * selected, p = softmax over them.
 *   dprob      DEVICE float[T,k]: gradient of the loss w.r.t. topk_prob
 *              (e.g. moe_bwd_dgrad_dprob's output)
 *   x          DEVICE [T,D] storage dtype (the layer input)
 *   w_router   DEVICE [E,D] storage dtype, row e = expert e's router vector
 *   dlogits    DEVICE float[T,E] output: p_j (dprob_j - sum_i p_i dprob_i) at
 *              the selected experts (sum over i ascending, float32), 0 elsewhere
 *   dw_router  DEVICE float[E,D] output: dlogits^T x.  Deterministic mode sums
 *              each expert's routed rows (routing order) in PH fixed row
 *              phases and adds the phase sums in phase order (PH = 8 when
 *              T*k/E < 512 and D is a multiple of 256, else 64); atomic mode
 *              adds the phase sums with atomicAdd (the nondeterministic control)
 *   dx_router  DEVICE [T,D] storage dtype output: dlogits wr, j ascending,
 *              float32 accumulation, one rounding (the router's share of dx;
 *              the caller adds it to the expert path's dx)
 * routing: topk_idx, topk_prob, counts, offsets and row_tok as written by
 * moe_fwd of the same problem.  Only the full layer is supported (combine = 1,
 * num_local = num_experts), since dw_router needs every expert's rows:
 * MOE_ERR_SHAPE otherwise.  Every output element is written.  Errors:
 * MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_MODE before anything is
 * enqueued; MOE_ERR_HIP for a launch failure. */
moe_status moe_router_bwd(const moe_problem* p, const moe_routing* routing, const float* dprob,
                          const void* x, const void* w_router, float* dlogits, float* dw_router,
                          void* dx_router, moe_mode mode, void* stream);

/* NVFP4 block quantisation of a row-major [rows, cols] tensor, the second
 * low-precision form whose encoded values and scale buffers the pages
 * fingerprint (French article, section "Méthodologie de débogage du
 * non-déterminisme").  The pages do not define it; this follows NVIDIA's
 * public description: E2M1 element codes, an E4M3 scale per 16 consecutive
 * elements of a row, a float32 scale g for the tensor.  Decisions in float32:
 *   g = amax / 2688 (1 if that is 0);  block scale sb = E4M3(amax_block / (6 g));
 *   element code = E2M1(|v| / (value(sb) g)) with v's sign (0 if the divisor is 0);
 * E4M3 / E2M1 round to nearest, ties to the even code, saturating at 448 / 6.
 *   in            DEVICE float32 or bf16 [rows, cols], 16-byte aligned;
 *                 cols a multiple of 16; finite values
 *   codes         DEVICE uint8 [rows, cols/2] output, 4-byte aligned: element
 *                 2j in the low nibble of byte j, 2j+1 in the high nibble
 *   scales        DEVICE uint8 [rows, cols/16] output (E4M3 codes)
 *   global_scale  DEVICE float32 [1] output: g
 * Three launches on `stream`; every output byte is independent of the launch
 * order.  Errors: MOE_ERR_DTYPE, MOE_ERR_SHAPE, MOE_ERR_NULL before anything
 * is enqueued; MOE_ERR_HIP for a launch failure. */
moe_status moe_nvfp4_quantize(const void* in, moe_dtype dtype, int64_t rows, int64_t cols, uint8_t* codes,
                              uint8_t* scales, float* global_scale, uint64_t debug_shuffle_seed, void* stream);

/* MXFP8 grouped GEMM, the low-precision variant of the fc1 data gradient:
 *   dx_rows[r, :] = dequant(dh)[r, :] . dequant(W1_e)^T   (r a routed row of
 *                   local expert e; dequant = E4M3 code * E8M0 block scale)
 * through gfx950's v_mfma_scale_f32_32x32x64_f8f6f4, float32 accumulation
 * in a fixed k order (64 k per MFMA, slices ascending), one rounding to bf16.
 * The pages name MXFP8 runs and fingerprint their encoded values and scale
 * buffers (French article, section "Méthodologie de débogage du
 * non-déterminisme"); the format is OCP MX v1.0 (moe_mx_quantize).
 *   dh_codes / dh_scales  DEVICE uint8 [rows_cap, F] / [rows_cap, F/32]
 *                         (moe_mx_quantize of dh)
 *   w1_codes / w1_scales  DEVICE uint8 [num_local, D, F] / [num_local, D, F/32]
 *                         (moe_mx_quantize of W1 viewed as [num_local*D, F])
 *   dx_rows               DEVICE bf16 [rows_cap, D] output; rows < R written
 * routing: counts, offsets and sched as written by moe_fwd.  The problem must
 * be bf16 with F a multiple of 128 and at most 2048 (the tile's scales are
 * staged in LDS).  Errors: MOE_ERR_DTYPE, MOE_ERR_SHAPE, MOE_ERR_NULL before
 * anything is enqueued; MOE_ERR_HIP for a launch failure. */
moe_status moe_mx_dgrad_fc1(const moe_problem* p, const moe_routing* routing, const uint8_t* dh_codes,
                            const uint8_t* dh_scales, const uint8_t* w1_codes, const uint8_t* w1_scales,
                            void* dx_rows, void* stream);

/* MXFP8 grouped GEMM, the low-precision variant of the fc2 data gradient, with
 * the fused epilogue of moe_bwd_dgrad_dprob's first stage:
 *   G[r, :]  = dequant(dy)[row_tok[r], :] . dequant(W2_e)^T   (r a routed row
 *              of local expert e), float32 accumulation in a fixed k order
 *              (64 k per scaled MFMA, slices ascending);
 *   dprob[t, j] = sum_f G[r, f] relu(h[r, f])^2 for the row r of slot (t, j)
 *              (0 for slots routed to non-local experts);
 *   dh[r, :]    = bf16(2 p_r G[r, :] relu(h[r, :]))   (p_r = the row's topk_prob).
 * This is the layer backward of moe_bwd_dgrad_dprob with dy and W2 replaced
 * by their MXFP8 values; the pages name MXFP8 runs and fingerprint their
 * encoded values and scale buffers (French article, section "Méthodologie de
 * débogage du non-déterminisme"); format OCP MX v1.0 (moe_mx_quantize).
 *   dy_codes / dy_scales  DEVICE uint8 [T, D] / [T, D/32] (moe_mx_quantize of dy)
 *   w2_codes / w2_scales  DEVICE uint8 [num_local, F, D] / [num_local, F, D/32]
 *                         (moe_mx_quantize of W2 viewed as [num_local*F, D])
 *   h                     DEVICE bf16 [rows_cap, F], as saved by moe_fwd
 *   dprob                 DEVICE float32 [T, k] output
 *   dh                    DEVICE bf16 [rows_cap, F] output; rows < R written
 *   ws, ws_bytes          the dgrad workspace of moe_workspace_size (mode)
 *   mode                  MOE_DETERMINISTIC: per-(row, N-tile) partials in the
 *                         workspace, then the fixed-tree combine of
 *                         moe_bwd_dgrad_dprob (bits independent of scheduling);
 *                         MOE_ATOMIC: dprob zeroed, partials added with atomics
 * routing: as written by moe_fwd.  The problem must be bf16 with D at most
 * 2048 (the tile's scales are staged in LDS).  Errors: MOE_ERR_DTYPE,
 * MOE_ERR_SHAPE, MOE_ERR_MODE, MOE_ERR_NULL, MOE_ERR_WORKSPACE before anything
 * is enqueued; MOE_ERR_HIP for a launch failure. */
moe_status moe_mx_dgrad_fc2(const moe_problem* p, const moe_routing* routing, const uint8_t* dy_codes,
                            const uint8_t* dy_scales, const uint8_t* w2_codes, const uint8_t* w2_scales,
                            const void* h, float* dprob, void* dh, void* ws, size_t ws_bytes,
                            moe_mode mode, void* stream);

/* Router forward for a train step of the layer: logits[t,e] = sum over d
 * ascending of x[t,d] * w_router[e,d] in float32 fused multiply-adds, one
 * thread per logit (no reduction across threads, so bit-exact).  The router
 * form is the reading stated at moe_router_bwd.
 *   x         DEVICE [T,D] storage dtype;  w_router DEVICE [E,D] storage dtype
 *   logits    DEVICE float[T,E] output (the input of moe_fwd)
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE (the problem's checks)
 * before anything is enqueued; MOE_ERR_HIP for a launch failure. */
moe_status moe_router_fwd(const moe_problem* p, const void* x, const void* w_router, float* logits,
                          void* stream);

/* Plain SGD step on a full-precision master copy, with the runtime copy
 * rebuilt through the same conversion the layer uses ("Trillion-Parameter
 * Pretraining Goes Bitwise-Deterministic", section "Interpretation": keep a
 * full-precision source of truth and reconstruct the runtime representation
 * through the training's conversion path):
 *   master[i] = fma(-lr, grad[i], master[i])   (float32)
 *   runtime[i] = master[i] rounded to `dtype` (RNE for MOE_BF16, copy for MOE_F32)
 *   master    DEVICE float[n], updated in place;  grad DEVICE float[n]
 *   runtime   DEVICE [n] of `dtype`, output
 * Elementwise, so bit-exact.  Errors: MOE_ERR_DTYPE (dtype not F32/BF16),
 * MOE_ERR_SHAPE (n < 0 or n >= 2^40), MOE_ERR_NULL; MOE_ERR_HIP for a launch
 * failure. */
moe_status moe_sgd_step(float* master, const float* grad, int64_t n, float lr, void* runtime, moe_dtype dtype,
                        void* stream);

/* MXFP8 block quantisation: the encoded values and block scales that a
 * low-precision run fingerprints (French article, section "Méthodologie de
 * débogage du non-déterminisme": for MXFP8 the encoded values and the scale
 * buffers are fingerprinted).  Format: OCP Microscaling Formats (MX) v1.0,
 * E4M3 elements with an E8M0 scale per 32 consecutive elements of a row:
 *   se    = floor(log2(max |v| over the block)) - 8, clamped to [-127, 127]
 *           (-127 when the block's largest magnitude is 0 or subnormal)
 *   scale = se + 127 (E8M0 byte)
 *   code  = E4M3(v * 2^-se): nearest, ties to the even code, saturated at
 *           +-448 (0x7E / 0xFE), sign kept (-0 -> 0x80)
 *   in      DEVICE [rows, cols] of dtype (MOE_F32 or MOE_BF16), 16-byte aligned,
 *           finite values
 *   codes   DEVICE uint8 [rows, cols], 8-byte aligned, output
 *   scales  DEVICE uint8 [rows, cols/32], output
 *   debug_shuffle_seed  0, or a test-only seed that shuffles the launch order
 * Every output byte is exact (integer rounding of exact values), so the
 * outputs are bit-identical whatever the order.  Errors: MOE_ERR_DTYPE,
 * MOE_ERR_SHAPE (rows < 0, cols not a positive multiple of 32, more than
 * 2^40 elements, misaligned pointers), MOE_ERR_NULL; MOE_ERR_HIP for a
 * launch failure. */
moe_status moe_mx_quantize(const void* in, moe_dtype dtype, int64_t rows, int64_t cols, uint8_t* codes,
                           uint8_t* scales, uint64_t debug_shuffle_seed, void* stream);

/* MXFP8 block quantisation along the other axis: for each of `groups`
 * row-major [rows, cols] matrices, the E4M3 codes and E8M0 scales of its
 * transpose, i.e. a block is 32 consecutive ROWS of one column, and the
 * codes of column c form row c of the output.  Same encoding as
 * moe_mx_quantize (OCP MX v1.0).  This is the form the forward GEMMs read
 * the weights in, contiguous along the contraction (the d_model axis of W1,
 * the d_ffn axis of W2), as MXFP8 training keeps a copy quantised along each
 * axis a GEMM contracts (French article, section "Méthodologie de débogage
 * du non-déterminisme": MXFP8 runs fingerprint their encoded values and
 * scale buffers).
 *   in      DEVICE [groups, rows, cols] of dtype (MOE_F32 or MOE_BF16); rows a
 *           positive multiple of 32; finite values
 *   codes   DEVICE uint8 [groups, cols, rows], 16-byte aligned, output
 *   scales  DEVICE uint8 [groups, cols, rows/32], output
 * Every output byte is exact, so the outputs are bit-identical whatever the
 * order.  Errors: MOE_ERR_DTYPE, MOE_ERR_SHAPE (rows not a positive multiple
 * of 32, cols <= 0, more than 2^40 elements, misaligned codes), MOE_ERR_NULL;
 * MOE_ERR_HIP for a launch failure. */
moe_status moe_mx_quantize_t(const void* in, moe_dtype dtype, int64_t groups, int64_t rows, int64_t cols,
                             uint8_t* codes, uint8_t* scales, uint64_t debug_shuffle_seed, void* stream);

/* MXFP8 grouped GEMM, the low-precision variant of the forward's fc1:
 *   h[r, :]   = bf16(dequant(x)[row_tok[r], :] . dequant(W1_e^T)^T)   (r a
 *               routed row of local expert e), float32 accumulation in a fixed
 *               k order (64 k per scaled MFMA, slices ascending);
 *   act[r, :] = bf16(relu(h[r, :])^2) of the rounded h (the input of fc2).
 * Format and sources as moe_mx_quantize / moe_mx_quantize_t.
 *   x_codes / x_scales    DEVICE uint8 [T, D] / [T, D/32] (moe_mx_quantize of x)
 *   w1t_codes / w1t_scales DEVICE uint8 [num_local, F, D] / [num_local, F, D/32]
 *                         (moe_mx_quantize_t of W1 [num_local, D, F])
 *   h, act                DEVICE bf16 [rows_cap, F] outputs; rows < R written
 * routing: as written by moe_fwd (top-k, permutation and work list).  The
 * problem must be bf16 with D a multiple of 128 and at most 2048.  Errors:
 * MOE_ERR_DTYPE, MOE_ERR_SHAPE, MOE_ERR_NULL before anything is enqueued;
 * MOE_ERR_HIP for a launch failure. */
moe_status moe_mx_fwd_fc1(const moe_problem* p, const moe_routing* routing, const uint8_t* x_codes,
                          const uint8_t* x_scales, const uint8_t* w1t_codes, const uint8_t* w1t_scales, void* h,
                          void* act, void* stream);

/* MXFP8 grouped GEMM, the low-precision variant of the forward's fc2, with
 * the forward's combine:
 *   o[r, :] = bf16(dequant(act)[r, :] . dequant(W2_e^T)^T), float32
 *             accumulation in a fixed k order;
 *   combine=1: y_t = sum_j p_tj o_(t,j), slots j ascending, float32
 *             accumulation from 0, rounded once (MOE_DETERMINISTIC; MOE_ATOMIC:
 *             the scatter-add control); combine=0: the o rows.
 *   act_codes / act_scales DEVICE uint8 [rows_cap, F] / [rows_cap, F/32]
 *                         (moe_mx_quantize of moe_mx_fwd_fc1's act)
 *   w2t_codes / w2t_scales DEVICE uint8 [num_local, D, F] / [num_local, D, F/32]
 *                         (moe_mx_quantize_t of W2 [num_local, F, D])
 *   y_or_rows             DEVICE bf16 [T, D] (combine=1) or [rows_cap, D]
 *   ws, ws_bytes          the forward workspace of moe_workspace_size (mode)
 * The problem must be bf16 with F a multiple of 128 and at most 2048.
 * Errors: MOE_ERR_DTYPE, MOE_ERR_SHAPE, MOE_ERR_MODE, MOE_ERR_NULL,
 * MOE_ERR_WORKSPACE before anything is enqueued; MOE_ERR_HIP for a launch
 * failure. */
moe_status moe_mx_fwd_fc2(const moe_problem* p, const moe_routing* routing, const uint8_t* act_codes,
                          const uint8_t* act_scales, const uint8_t* w2t_codes, const uint8_t* w2t_scales,
                          void* y_or_rows, void* ws, size_t ws_bytes, moe_mode mode, void* stream);

/* Rows read by moe_mx_quantize_wgrad (cols: the operand's width). */
typedef enum moe_mxw_src {
  MOE_MXW_TOKEN = 0, /* src bf16 [T, D]: row r of the output is src[row_tok[r]] (x or dY), cols = D */
  MOE_MXW_ROW = 1,   /* src bf16 [rows_cap, F]: routed row r (dH), cols = F */
  MOE_MXW_ACT_P = 2  /* src bf16 h [rows_cap, F]: p_r relu(h_r)^2 formed in float32 (the
                        square rounded, then the product; relu(v) = v > 0 ? v : +0), cols = F */
} moe_mxw_src;

/* Padded rows of the MXFP8 weight-gradient operands for problem p:
 * rpad_cap = rows_cap + num_local * 63 rounded up to a multiple of 64 (each
 * expert's routed rows padded to a multiple of 64).  Errors: those of the
 * problem's validation, MOE_ERR_NULL. */
moe_status moe_mx_wgrad_rows(const moe_problem* p, int64_t* rpad_cap);

/* MXFP8 encoding of a weight-gradient operand, quantised along the routed
 * rows: the contraction axis of dW1_e = X_e^T dH_e and dW2_e = A_e^T dY_e
 * (A = p relu(h)^2; the English digest's backward of the expert MLP), so
 * that a block scale is constant along each product.  The format is
 * moe_mx_quantize's (the French article, section on the method for
 * debugging non-determinism, fingerprints the encoded values and the scale
 * buffers; OCP MX v1.0: E4M3 codes, one E8M0 scale per 32 elements).
 * Layout: expert e owns padded rows poff[e] .. poff[e+1], poff the prefix
 * sum of its routed row counts rounded up to a multiple of 64; padded row
 * poff[e] + i is its routed row offsets[e] + i for i below its count, and
 * zeros past it.  A block is 32 consecutive padded rows of one column, so
 * blocks start at an expert's first row.  Codes and scales are stored
 * slice-major: the 64 codes and two scales of column c in 64-row slice j
 * are codes[j][c][0..63] and scales[j][c][0..1] (slices outermost, columns
 * side by side), so that the GEMM reads a tile's slice as one contiguous
 * run.
 *   src            DEVICE bf16, as moe_mxw_src describes, 16-byte aligned
 *   codes          DEVICE uint8 [rpad_cap / 64, cols, 64], 16-byte aligned
 *   scales         DEVICE uint8 [rpad_cap / 64, cols, 2]
 * Slices from poff[num_local] / 64 on are not written.  routing: as written by
 * moe_fwd.  The problem must be bf16 with max(D, F) * (T rounded up to 64)
 * < 2^31 (one expert's encodings, which can hold every token).
 * Deterministic: every byte depends on the inputs only.  Errors:
 * MOE_ERR_DTYPE, MOE_ERR_SHAPE (sizes, alignment, kind), MOE_ERR_NULL before
 * anything is enqueued; MOE_ERR_HIP for a launch failure. */
moe_status moe_mx_quantize_wgrad(const moe_problem* p, const moe_routing* routing, const void* src,
                                 moe_mxw_src kind, uint8_t* codes, uint8_t* scales, void* stream);

/* MXFP8 weight gradients, both matrices, from operands encoded by
 * moe_mx_quantize_wgrad (x: MOE_MXW_TOKEN of X, dh: MOE_MXW_ROW of dH,
 * act: MOE_MXW_ACT_P of h, dy: MOE_MXW_TOKEN of dY):
 *   dW1[e] = dequant(x_e) . dequant(dh_e)^T   [D, F] per local expert,
 *   dW2[e] = dequant(act_e) . dequant(dy_e)^T [F, D],
 * over expert e's padded rows.  Each output tile is accumulated in
 * float32 by one workgroup over all of the expert's rows in a fixed order
 * (64 rows per scaled MFMA, ascending) and stored once: the result is
 * bitwise reproducible with no reduction step (there is no atomic mode).
 * An expert without rows gets zeros.
 *   *_codes        DEVICE uint8 [rpad_cap / 64, D or F, 64], 16-byte aligned
 *   *_scales       DEVICE uint8 [rpad_cap / 64, D or F, 2], 16-byte aligned
 *   dw1, dw2       DEVICE float32 [num_local, D, F] / [num_local, F, D]
 * The problem must be bf16 with max(D, F) * (T rounded up to 64) < 2^31.
 * Errors:
 * MOE_ERR_DTYPE, MOE_ERR_SHAPE, MOE_ERR_NULL before anything is enqueued;
 * MOE_ERR_HIP for a launch failure. */
moe_status moe_mx_wgrad(const moe_problem* p, const moe_routing* routing, const uint8_t* x_codes,
                        const uint8_t* x_scales, const uint8_t* dh_codes, const uint8_t* dh_scales,
                        const uint8_t* act_codes, const uint8_t* act_scales, const uint8_t* dy_codes,
                        const uint8_t* dy_scales, float* dw1, float* dw2, void* stream);

/* Diagnostic for the measurement of the percent of bf16 dense peak: the
 * attainable MFMA rate of the device.  Enqueues on `stream` one launch of
 * `blocks` workgroups of 4 waves; every wave issues iters x 8 independent
 * v_mfma_f32_32x32x16_bf16 on register operands that hold `value` in every
 * element (no memory traffic in the loop), then thread t of block b writes
 * the sum of its 128 accumulator elements to sink[256 b + t].  The launch
 * performs blocks * 4 * iters * 8 * 32768 floating-point operations; the
 * caller times it with events on the same stream.  Each sink element is
 * 2048 * value^2 * iters while that is exact in float32.
 *   blocks  1 .. 2^31-1 (two per compute unit fill every SIMD twice)
 *   iters   >= 1
 *   value   a float whose low 16 bits are zero (a bf16 value)
 *   sink    DEVICE float[256 * blocks], caller-owned
 * Errors: MOE_ERR_SHAPE (blocks, iters or value out of range), MOE_ERR_NULL
 * (sink), MOE_ERR_HIP (launch failure).  Nothing is enqueued on error. */
moe_status moe_mfma_rate(int64_t blocks, int64_t iters, float value, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEDET_H */
