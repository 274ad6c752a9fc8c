// Router top-k + softmax and the stable token permutation (counting sort by
// local expert), integer-exact.
//
// Readings of the pages (which give no router details): experts are ranked
// by descending float32 logit, equal logits go to the lower expert index
// (-0.0 compares equal to +0.0), and the routing probabilities are the
// softmax over the k selected logits.  The permutation is stable in the flat
// slot index t*k+j, so the row order inside an expert -- the K order of the
// weight-gradient reduction -- is fixed by the routing alone.
//
//  route_kernel    one wave per token at a time (8 waves per chunk of 16
//                  tokens, two tokens each): k rounds of a wave-wide argmax,
//                  then the softmax; per-chunk histogram of local experts in
//                  LDS (integer atomics: exact in any order).
//  scan_kernel     per-expert exclusive bases of every chunk and the expert
//                  offsets (one workgroup; each expert's chunks split over
//                  several threads, their loads issued in batches).
//  scatter_kernel  one wave per chunk walks its slots in order, 64 at a
//                  time; a lane's rank among equal experts comes from ballots,
//                  so the result is the stable order.  Atomic mode claims rows
//                  with global atomics instead (order not fixed).
#include "common.h"
#include "kernels.h"

namespace moedet {

namespace {

// Candidate (logit v, expert e) as one unsigned 64-bit key, larger = better:
// the high word orders floats (-0.0 taken as +0.0, so the two compare equal),
// the low word is ~e (a lower expert wins a tie).  0 stands for "none": every
// finite or infinite logit maps above it.  A single unsigned comparison then
// decides, without branches.
DEV uint64_t cand_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  const uint32_t s = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)s << 32) | (uint32_t)~e;
}
DEV float key_value(uint64_t key) {
  const uint32_t s = (uint32_t)(key >> 32);
  return __uint_as_float((s & 0x80000000u) ? (s & 0x7fffffffu) : ~s);
}
DEV int key_expert(uint64_t key) { return (int)~(uint32_t)key; }

}  // namespace

// PER logits per lane (E <= 64 * PER); kRouteWaves waves per chunk of
// kRouteChunk tokens, one token per wave at a time.
constexpr int kRouteWaves = 8;
template <int PER>
__global__ __launch_bounds__(kRouteWaves * 64) void route_kernel(RouteParams P) {
  __shared__ int s_hist[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t b = blockIdx.x;  // chunk index (fixed: the histogram is per chunk)
  if (P.seed) shuffle_delay(P.seed, b);
  for (int i = tid; i < P.el; i += kRouteWaves * 64) s_hist[i] = 0;
  __syncthreads();
  const int E = P.E, k = P.k;
  for (int tt = w; tt < kRouteChunk; tt += kRouteWaves) {
    const int64_t t = b * kRouteChunk + tt;
    if (t >= P.T) break;
    const float* row = P.logits + t * E;
    // this lane's candidates; taken ones are set to 0 (none)
    uint64_t key[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + kWave * i;
      key[i] = e < E ? cand_key(row[e], e) : 0ull;
    }
    float vmax = 0.f, my_v = 0.f;
    int my_e = -1;
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0ull;
#pragma unroll
      for (int i = 0; i < PER; ++i) best = key[i] > best ? key[i] : best;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t o = ((uint64_t)(uint32_t)__shfl_xor((int)(best >> 32), off, 64) << 32) |
                           (uint32_t)__shfl_xor((int)(uint32_t)best, off, 64);
        best = o > best ? o : best;
      }
      // best is identical in every lane (the keys are distinct)
      const int be = key_expert(best);
      const float bv = key_value(best);
      if ((be & (kWave - 1)) == lane) {
#pragma unroll
        for (int i = 0; i < PER; ++i)
          if (i == be / kWave) key[i] = 0ull;
      }
      if (j == 0) vmax = bv;
      if (lane == j) {
        my_v = bv;
        my_e = be;
      }
    }
    float ex = lane < k ? expf(my_v - vmax) : 0.f;
    float sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum = sum + __shfl_xor(sum, off, 64);
    if (lane < k) {
      P.topk_idx[t * k + lane] = my_e;
      P.topk_prob[t * k + lane] = ex / sum;
      const int le = my_e - P.eb;
      if (le >= 0 && le < P.el) atomicAdd(&s_hist[le], 1);
    }
  }
  __syncthreads();
  for (int i = tid; i < P.el; i += kRouteWaves * 64) P.hist[b * P.el + i] = s_hist[i];
}

// Row tiles of height BM over the experts' rows, longest first: the full
// tiles expert-major, then the partial tiles by descending rows (bitonic sort
// of (BM - rows) << 10 | expert).  Entries {expert, first row in the expert,
// first row overall, rows}; returns the count (uniform).  One thread per
// expert (e = threadIdx.x) with its row count `total` and offset `off_e`.
DEV int row_tile_list(const RouteParams& P, int4* mt, int BM, const int* s_cnt, const int* s_off, int* s_pre,
                      int* s_tmp, uint32_t* s_key, int total, int off_e) {
  const int e = threadIdx.x;
  block_exclusive_scan<1024>(s_pre, s_tmp, P.el, [&](int g) { return s_cnt[g] / BM; });
  const int nfull = s_pre[P.el];
  if (e < P.el)
    for (int i = 0; i < total / BM; ++i) mt[s_pre[e] + i] = int4{e, i * BM, off_e + i * BM, BM};
  s_key[e] = (e < P.el && total % BM) ? ((uint32_t)(BM - total % BM) << 10) | (uint32_t)e : 0xffffffffu;
  __syncthreads();
  // bitonic sort of the first N = next_pow2(el) keys (the rest are sentinels
  // already in place)
  int N = 1;
  while (N < P.el) N <<= 1;
  for (int k = 2; k <= N; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int o = e ^ j;
      if (e < N && o > e) {
        const uint32_t a = s_key[e], b = s_key[o];
        if ((a > b) == ((e & k) == 0)) {
          s_key[e] = b;
          s_key[o] = a;
        }
      }
      __syncthreads();
    }
  const uint32_t key = s_key[e];
  if (key != 0xffffffffu) {
    const int g = (int)(key & 1023u);
    const int c = s_cnt[g];
    const int m0 = c / BM * BM;
    mt[nfull + e] = int4{g, m0, s_off[g] + m0, c - m0};
  }
  __syncthreads();
  // number of partial tiles = sorted keys below the sentinel
  block_exclusive_scan<1024>(s_pre, s_tmp, P.el, [&](int g) { return s_cnt[g] % BM != 0 ? 1 : 0; });
  const int n = nfull + s_pre[P.el];
  __syncthreads();
  return n;
}

// hist[c][e] -> exclusive row base of chunk c for expert e; counts, offsets;
// then the backward work list (routing.sched), from counts alone:
//   row tiles of bm and of bm2 rows (row_tile_list): every expert's full
//   tiles (expert-major), then the partial last tiles ordered by descending
//   rows (ties by expert), so that a GEMM whose tiles outnumber the compute
//   units leaves the smallest tiles for its last round;
//   weight-gradient units: expert g in S_g = max(1, ceil(cnt_g / kc)) chunks,
//   chunk s covering rows [s cnt/S, (s+1) cnt/S); chunks s >= 1 of a split
//   expert own partial slot sum_{g'<g} (S_g' - 1) + s - 1; the side table
//   holds {S_g, s, sum_{g'<g} (S_g' - 1), 0} for the ordered reduction.
__global__ __launch_bounds__(1024) void permute_scan_kernel(RouteParams P) {
  __shared__ int s_pre[kMaxExperts + 1];
  __shared__ int s_tmp[16];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_off[kMaxExperts];
  __shared__ uint32_t s_key[1024];
  __shared__ int s_part[1024];
  __shared__ int s_ppre[1025];
  const int e = threadIdx.x;
  // Chunk counts hist[c][g] -> row bases: expert g's chunks are split over
  // tpe threads (the largest power of two with tpe * el <= 1024), thread
  // (g, part) taking a contiguous range.  Pass 1 sums each range; the ranges'
  // exclusive prefix within the expert and the experts' offsets follow; pass
  // 2 writes offsets[g] + (rows of g in earlier chunks) into hist.  Loads
  // are issued 16 at a time.  Integer sums: exact in any grouping.
  int tpe = 1;
  while (tpe * 2 * P.el <= 1024) tpe *= 2;
  const int g = e / tpe, part = e % tpe;
  const bool active = g < P.el;
  const int per = (P.nchunk + tpe - 1) / tpe;
  const int c0 = min(P.nchunk, part * per), c1 = min(P.nchunk, c0 + per);
  constexpr int kBatch = 16;
  int sum = 0;
  if (active) {
    for (int c = c0; c < c1; c += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) v[q] = P.hist[(int64_t)min(c + q, c1 - 1) * P.el + g];  // branch-free
#pragma unroll
      for (int q = 0; q < kBatch; ++q) sum += c + q < c1 ? v[q] : 0;
    }
  }
  s_part[e] = sum;
  __syncthreads();
  // prefix over the (expert, range) sums in that order: an expert's total
  // and each range's offset inside its expert are differences of it
  block_exclusive_scan<1024>(s_ppre, s_tmp, 1024, [&](int x) { return s_part[x]; });
  int total = 0;  // rows of expert e (thread e as an expert from here on)
  if (e < P.el) {
    total = s_ppre[(e + 1) * tpe] - s_ppre[e * tpe];
    P.counts[e] = total;
    s_cnt[e] = total;
  }
  block_exclusive_scan<1024>(s_pre, s_tmp, P.el, [&](int x) { return s_cnt[x]; });
  // el may be the block size (1024): thread 0 also writes the total
  if (e < P.el) P.offsets[e] = s_pre[e];
  if (e == 0) P.offsets[P.el] = s_pre[P.el];
  const int off_e = e < P.el ? s_pre[e] : 0;
  if (e < P.el) {
    s_off[e] = off_e;
    if (P.atomic) P.cursor[e] = off_e;
  }
  if (active) {
    int run = s_pre[g] + (s_ppre[e] - s_ppre[g * tpe]);
    for (int c = c0; c < c1; c += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) v[q] = P.hist[(int64_t)min(c + q, c1 - 1) * P.el + g];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        if (c + q < c1) P.hist[(int64_t)(c + q) * P.el + g] = run;
        run += v[q];
      }
    }
  }
  __syncthreads();

  // row tiles of height P.bm (header word 0) and P.bm2 (header word 2)
  const int n1 = row_tile_list(P, (int4*)(P.sched + kSchedHeader), P.bm, s_cnt, s_off, s_pre, s_tmp, s_key, total, off_e);
  const int n2 = row_tile_list(P, (int4*)(P.sched + P.list2_at), P.bm2, s_cnt, s_off, s_pre, s_tmp, s_key, total, off_e);
  if (e == 0) {
    P.sched[0] = n1;
    P.sched[2] = n2;
    P.sched[3] = 0;
  }
  __syncthreads();
  // weight-gradient units: one packed scan of (S << 16 | (S - 1))
  const int kc = P.kc;
  auto nsplit = [&](int g) { const int c = s_cnt[g]; return c > kc ? (c + kc - 1) / kc : 1; };
  block_exclusive_scan<1024>(s_pre, s_tmp, P.el, [&](int g) { return nsplit(g); });
  const int ubase = e < P.el ? s_pre[e] : 0;
  const int nunits = s_pre[P.el];
  __syncthreads();
  block_exclusive_scan<1024>(s_pre, s_tmp, P.el, [&](int g) { return nsplit(g) - 1; });
  if (e < P.el) {
    int4* wu = (int4*)(P.sched + kSchedHeader) + P.mt_cap;
    int4* aux = (int4*)(P.sched + P.aux_at);
    const int S = nsplit(e);
    for (int sc = 0; sc < S; ++sc) {
      const int lo = (int)((int64_t)sc * total / S), hi = (int)((int64_t)(sc + 1) * total / S);
      wu[ubase + sc] = int4{e | (S > 1 ? 1 << 30 : 0), off_e + lo, hi - lo, sc > 0 ? s_pre[e] + sc - 1 : -1};
      aux[ubase + sc] = int4{S, sc, s_pre[e], 0};
    }
  }
  if (e == 0) P.sched[1] = nunits;
  __syncthreads();
  // padded row offsets of the MXFP8 weight-gradient operands
  block_exclusive_scan<1024>(s_pre, s_tmp, P.el, [&](int g) { return (s_cnt[g] + kMxPad - 1) / kMxPad * kMxPad; });
  if (e < P.el) P.sched[P.pad_at + e] = s_pre[e];
  if (e == 0) P.sched[P.pad_at + P.el] = s_pre[P.el];
}

__global__ __launch_bounds__(64) void permute_scatter_kernel(RouteParams P) {
  __shared__ int s_base[kMaxExperts];
  const int lane = threadIdx.x;
  const int64_t c = blockIdx.x;
  if (P.seed) shuffle_delay(P.seed, c);
  for (int e = lane; e < P.el; e += 64) s_base[e] = P.hist[c * P.el + e];
  __syncthreads();
  const int k = P.k;
  const int64_t i_begin = c * kRouteChunk * k;
  const int64_t i_end = min((c + 1) * kRouteChunk, P.T) * k;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  for (int64_t g0 = i_begin; g0 < i_end; g0 += 64) {
    const int64_t i = g0 + lane;
    const bool valid = i < i_end;
    const int e = valid ? P.topk_idx[i] - P.eb : -1;
    const bool loc = valid && e >= 0 && e < P.el;
    int row = -1;
    if (!P.atomic) {
      uint64_t match = __ballot(loc);
#pragma unroll
      for (int bit = 0; bit < 10; ++bit) {
        const bool my = (e >> bit) & 1;
        const uint64_t m = __ballot(loc && my);
        match &= my ? m : ~m;
      }
      const int rank = __popcll(match & lt_mask);
      const int cnt = __popcll(match);
      const int base = loc ? s_base[e] : 0;
      __syncthreads();
      if (loc && rank == 0) s_base[e] = base + cnt;
      __syncthreads();
      if (loc) row = base + rank;
    } else if (loc) {
      row = atomicAdd(&P.cursor[e], 1);
    }
    if (valid) P.slot_row[i] = loc ? row : -1;
    if (loc) {
      P.row_src[row] = (int32_t)i;
      P.row_tok[row] = (int32_t)(i / k);
      P.row_prob[row] = P.topk_prob[i];
    }
  }
}

hipError_t launch_route(const RouteParams& P, hipStream_t st) {
  if (P.nchunk <= 0) return hipSuccess;
  const dim3 blk(kRouteWaves * 64);
  if (P.E <= 64)
    route_kernel<1><<<P.nchunk, blk, 0, st>>>(P);
  else if (P.E <= 128)
    route_kernel<2><<<P.nchunk, blk, 0, st>>>(P);
  else if (P.E <= 256)
    route_kernel<4><<<P.nchunk, blk, 0, st>>>(P);
  else if (P.E <= 512)
    route_kernel<8><<<P.nchunk, blk, 0, st>>>(P);
  else
    route_kernel<kMaxExperts / kWave><<<P.nchunk, blk, 0, st>>>(P);
  return hipGetLastError();
}

hipError_t launch_permute_scan(const RouteParams& P, hipStream_t st) {
  permute_scan_kernel<<<1, 1024, 0, st>>>(P);
  return hipGetLastError();
}

hipError_t launch_permute_scatter(const RouteParams& P, hipStream_t st) {
  if (P.nchunk <= 0) return hipSuccess;
  permute_scatter_kernel<<<P.nchunk, 64, 0, st>>>(P);
  return hipGetLastError();
}

}  // namespace moedet
