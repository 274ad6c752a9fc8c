// Expert grouped GEMMs for gfx950.
//
//  rowgemm  C[rows of expert g, N] = A[rows, K] * B_g, K = D or F.
//           fc1 forward (x gathered, W1 [D][F]), fc2 forward (relu(h)^2,
//           W2 [F][D]), fc2 dgrad (dy gathered, W2 read as [N=F][K=D]) with
//           the dprob / dh epilogue, fc1 dgrad (dh, W1 read as [N=D][K=F]).
//  wgrad    dW_g[M, N] = sum over the expert's rows of A_row^T B_row, the
//           rows split into chunks whose size depends on shapes only.
//
// Expert row counts live on the device, so every workgroup derives the
// work decomposition itself from counts[] (no host synchronisation); the
// grid is an upper bound and surplus workgroups exit at once.
//
// Deterministic reductions (the English digest "Trillion-Parameter
// Pretraining Goes Bitwise-Deterministic", section "Interpretation"):
//  * dprob: each (row, N-tile) pair writes its own float32 partial; a
//    later pass adds the partials in N-tile order.  The atomic mode adds
//    them into dprob[token] directly, in arrival order.
//  * wgrad split-K: chunk partials go to the output (chunk 0) and to
//    workspace slots (chunks 1..S-1) and a later pass adds them in chunk
//    order; the atomic mode adds all chunks atomically into a zeroed dW.
#include "gemm.h"
#include "kernels.h"

namespace moedet {

// ---------------------------------------------------------------- rowgemm
template <typename T, bool A_ACT, bool B_MNC, int EPI>
__global__ __launch_bounds__(256) void rowgemm_kernel(RowGemmParams P) {
  using C = Tile<T>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  __shared__ int s_pre[kMaxExperts + 1];
  __shared__ int s_tmp[8];
  T* As0 = (T*)smem;
  T* Bs0 = As0 + 2 * C::OPER_ELEMS;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int G = P.groups;
  const int nN = P.N / C::BN;

  block_exclusive_scan<256>(s_pre, s_tmp, G, [&](int g) { return (P.counts[g] + C::BM - 1) / C::BM; });
  const int64_t U = (int64_t)s_pre[G] * nN;
  const int64_t L = map_unit(blockIdx.x, U, P.seed);
  if (L < 0) return;
  const int64_t mt_all = L / nN;
  const int nt = (int)(L % nN);
  const int g = find_group(s_pre, G, mt_all);
  const int m0 = (int)(mt_all - s_pre[g]) * C::BM;
  const int n0 = nt * C::BN;
  const int cnt = P.counts[g];
  const int64_t off = P.offsets[g];
  const int mvalid = min(C::BM, cnt - m0);

  // A rows: global rows off+m0 .. (gathered through a_rows when given)
  KcLoader<T, A_ACT> la;
  la.init(tid, (const T*)P.a, P.lda, P.a_rows, off + m0, mvalid, P.a_rows != nullptr);
  const T* Bg = (const T*)P.b + (int64_t)g * P.b_gstride;

  f32x16_t acc[C::MB][C::NB];
  zero_acc<T>(acc);
  const int nsteps = P.K / C::BK;

  if constexpr (!B_MNC) {
    KcLoader<T, false> lb;
    lb.init(tid, Bg, P.ldb, nullptr, n0, C::BN, false);
    la.load(0);
    lb.load(0);
    la.store(As0, tid);
    lb.store(Bs0, tid);
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
      const int cur = s & 1;
      if (s + 1 < nsteps) {
        la.load((int64_t)(s + 1) * C::BK);
        lb.load((int64_t)(s + 1) * C::BK);
      }
      mma_slice<T>(As0 + cur * C::OPER_ELEMS, Bs0 + cur * C::OPER_ELEMS, acc, wm, wn, lane);
      if (s + 1 < nsteps) {
        la.store(As0 + (cur ^ 1) * C::OPER_ELEMS, tid);
        lb.store(Bs0 + (cur ^ 1) * C::OPER_ELEMS, tid);
      }
      __syncthreads();
    }
  } else {
    // B_g stored [K][N]: K row k of slice s is Bg + (s*BK + k)*ldb + n0.
    MncLoader<T, false, false> lb;
    auto none = [](int) { return 1.f; };
    auto rows_of = [&](int s) {
      return [=](int k) { return Bg + ((int64_t)s * C::BK + k) * P.ldb + n0; };
    };
    la.load(0);
    lb.load(tid, rows_of(0), none);
    la.store(As0, tid);
    lb.store(Bs0, tid);
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
      const int cur = s & 1;
      if (s + 1 < nsteps) {
        la.load((int64_t)(s + 1) * C::BK);
        lb.load(tid, rows_of(s + 1), none);
      }
      mma_slice<T>(As0 + cur * C::OPER_ELEMS, Bs0 + cur * C::OPER_ELEMS, acc, wm, wn, lane);
      if (s + 1 < nsteps) {
        la.store(As0 + (cur ^ 1) * C::OPER_ELEMS, tid);
        lb.store(Bs0 + (cur ^ 1) * C::OPER_ELEMS, tid);
      }
      __syncthreads();
    }
  }

  // ------------------------------------------------------------ epilogue
  const int r32 = lane & 31, half = lane >> 5;
  const int WTM = C::BM / C::WM, WTN = C::BN / C::WN;
  if constexpr (EPI == kEpiStore) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      const int m = wm * WTM + mb * 32 + r32;
      if (m >= mvalid) continue;
      T* crow = (T*)P.c + (off + m0 + m) * P.ldc + n0 + wn * WTN;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = nb * 32 + 8 * i + 4 * half;
          const f32x16_t& a = acc[mb][nb];
          if constexpr (sizeof(T) == 2) {
            u32x2_t v = {pack_bf16x2(a[4 * i], a[4 * i + 1]), pack_bf16x2(a[4 * i + 2], a[4 * i + 3])};
            *(u32x2_t*)(crow + n) = v;
          } else {
            *(f32x4_t*)(crow + n) = f32x4_t{a[4 * i], a[4 * i + 1], a[4 * i + 2], a[4 * i + 3]};
          }
        }
    }
  } else {
    // fc2 dgrad: acc = G = dy W2^T for rows m, columns f of this N-tile.
    //   part[row][nt] = sum_f G * relu(h)^2   (fixed order: nb, i, q within
    //                   a lane; then the lane pair; then wave wn = 0, 1)
    //   dh = (2 p G) * relu(h)
    float* s_part = (float*)smem;  // [WN][BM], operand buffers are free now
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
      const int m = wm * WTM + mb * 32 + r32;
      const bool valid = m < mvalid;
      const int64_t grow = off + m0 + m;
      float part = 0.f;
      if (valid) {
        const float p2 = 2.f * P.row_prob[grow];
        const T* hrow = (const T*)P.h + grow * P.ldh + n0 + wn * WTN;
        T* drow = (T*)P.c + grow * P.ldc + n0 + wn * WTN;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = nb * 32 + 8 * i + 4 * half;
            const f32x16_t& a = acc[mb][nb];
            float hv[4];
            if constexpr (sizeof(T) == 2) {
              u32x2_t hh = *(const u32x2_t*)(hrow + n);
              hv[0] = bf16_to_f32(hh[0] & 0xffffu);
              hv[1] = bf16_to_f32(hh[0] >> 16);
              hv[2] = bf16_to_f32(hh[1] & 0xffffu);
              hv[3] = bf16_to_f32(hh[1] >> 16);
            } else {
              f32x4_t hh = *(const f32x4_t*)(hrow + n);
              hv[0] = hh[0]; hv[1] = hh[1]; hv[2] = hh[2]; hv[3] = hh[3];
            }
            float dh[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float gq = a[4 * i + q];
              const float rh = relu(hv[q]);
              part = __builtin_fmaf(gq, rh * rh, part);
              dh[q] = (p2 * gq) * rh;
            }
            if constexpr (sizeof(T) == 2) {
              *(u32x2_t*)(drow + n) = u32x2_t{pack_bf16x2(dh[0], dh[1]), pack_bf16x2(dh[2], dh[3])};
            } else {
              *(f32x4_t*)(drow + n) = f32x4_t{dh[0], dh[1], dh[2], dh[3]};
            }
          }
      }
      // lanes l and l^32 hold the two column halves of the same row;
      // a + b == b + a, so both get the same bits.
      part = part + __shfl_xor(part, 32, 64);
      if (half == 0) s_part[wn * C::BM + m] = part;
    }
    __syncthreads();
    for (int m = tid; m < mvalid; m += 256) {
      float v = s_part[m];
#pragma unroll
      for (int w = 1; w < C::WN; ++w) v = v + s_part[w * C::BM + m];
      const int64_t grow = off + m0 + m;
      if (P.atomic)
        atomicAdd(P.dprob + P.row_src[grow], v);
      else
        P.part[grow * P.n_tiles + nt] = v;
    }
  }
}

// ---------------------------------------------------------------- wgrad
template <typename T, bool A_GATHER, bool A_ACT, bool B_GATHER, bool B_SCALE>
__global__ __launch_bounds__(256) void wgrad_kernel(WgradParams P) {
  using C = Tile<T>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  __shared__ int s_tok[kMaxChunkRows];
  __shared__ float s_prob[B_SCALE ? kMaxChunkRows : 1];
  T* As0 = (T*)smem;
  T* Bs0 = As0 + 2 * C::OPER_ELEMS;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int G = P.groups;
  const int nN = P.N / C::BN;
  const int tiles = (P.M / C::BM) * nN;
  const int32_t* unit_start = P.sched;
  const int32_t* slot_base = P.sched + (G + 1);

  const int64_t U = (int64_t)unit_start[G] * tiles;
  const int64_t L = map_unit(blockIdx.x, U, P.seed);
  if (L < 0) return;
  const int64_t u = L / tiles;
  const int tile = (int)(L % tiles);
  const int g = find_group(unit_start, G, u);
  const int s = (int)(u - unit_start[g]);
  const int cnt = P.counts[g];
  const int S = cnt > P.kc ? (cnt + P.kc - 1) / P.kc : 1;
  const int k_lo = (int)((int64_t)s * cnt / S), k_hi = (int)((int64_t)(s + 1) * cnt / S);
  const int klen = k_hi - k_lo;
  const int64_t row0 = (int64_t)P.offsets[g] + k_lo;
  const int m0 = (tile / nN) * C::BM, n0 = (tile % nN) * C::BN;

  for (int i = tid; i < klen; i += 256) {
    s_tok[i] = (A_GATHER || B_GATHER) ? P.row_tok[row0 + i] : 0;
    if constexpr (B_SCALE) s_prob[i] = P.row_prob[row0 + i];
  }
  __syncthreads();

  f32x16_t acc[C::MB][C::NB];
  zero_acc<T>(acc);
  const int nsteps = (klen + C::BK - 1) / C::BK;

  MncLoader<T, A_ACT, false> la;
  MncLoader<T, false, B_SCALE> lb;
  const T* Ab = (const T*)P.a;
  const T* Bb = (const T*)P.b;
  auto a_rows = [&](int st) {
    return [=](int k) -> const T* {
      const int kk = st * C::BK + k;
      if (kk >= klen) return nullptr;
      const int64_t r = A_GATHER ? (int64_t)s_tok[kk] : row0 + kk;
      return Ab + r * P.lda + m0;
    };
  };
  auto b_rows = [&](int st) {
    return [=](int k) -> const T* {
      const int kk = st * C::BK + k;
      if (kk >= klen) return nullptr;
      const int64_t r = B_GATHER ? (int64_t)s_tok[kk] : row0 + kk;
      return Bb + r * P.ldb + n0;
    };
  };
  auto no_scale = [](int) { return 1.f; };
  auto b_scale = [&](int st) {
    return [=](int k) { return B_SCALE ? s_prob[st * C::BK + k] : 1.f; };
  };

  if (nsteps > 0) {
    la.load(tid, a_rows(0), no_scale);
    lb.load(tid, b_rows(0), b_scale(0));
    la.store(As0, tid);
    lb.store(Bs0, tid);
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
      const int cur = st & 1;
      if (st + 1 < nsteps) {
        la.load(tid, a_rows(st + 1), no_scale);
        lb.load(tid, b_rows(st + 1), b_scale(st + 1));
      }
      mma_slice<T>(As0 + cur * C::OPER_ELEMS, Bs0 + cur * C::OPER_ELEMS, acc, wm, wn, lane);
      if (st + 1 < nsteps) {
        la.store(As0 + (cur ^ 1) * C::OPER_ELEMS, tid);
        lb.store(Bs0 + (cur ^ 1) * C::OPER_ELEMS, tid);
      }
      __syncthreads();
    }
  }

  // Destination: a single chunk (or chunk 0) writes dW directly; chunks
  // 1..S-1 write workspace slots in det mode, or add atomically.
  const bool atomic_add = P.atomic && S > 1;
  float* dst = P.dw + (int64_t)g * P.M * P.N;
  if (!P.atomic && s > 0) dst = P.slots + (int64_t)(slot_base[g] + s - 1) * P.M * P.N;
  const int r32 = lane & 31, half = lane >> 5;
  const int WTM = C::BM / C::WM, WTN = C::BN / C::WN;
#pragma unroll
  for (int mb = 0; mb < C::MB; ++mb) {
    const int m = m0 + wm * WTM + mb * 32 + r32;
    float* crow = dst + (int64_t)m * P.N + n0 + wn * WTN;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
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

// Schedule for wgrad: unit_start[g] = sum_{g'<g} S_g' and slot_base[g] =
// sum_{g'<g} (S_g' - 1), S_g = max(1, ceil(cnt_g / kc)).  Atomic mode also
// zeroes dW of every expert that is split (S_g >= 2).
__global__ __launch_bounds__(256) void wgrad_prep_kernel(WgradPrepParams P) {
  __shared__ int s_pre[kMaxExperts + 1];
  __shared__ int s_tmp[8];
  const int G = P.groups;
  auto nsplit = [&](int g) {
    const int c = P.counts[g];
    return c > P.kc ? (c + P.kc - 1) / P.kc : 1;
  };
  if (blockIdx.x == 0) {
    block_exclusive_scan<256>(s_pre, s_tmp, G, nsplit);
    for (int g = threadIdx.x; g <= G; g += 256) P.sched[g] = s_pre[g];
    __syncthreads();
    block_exclusive_scan<256>(s_pre, s_tmp, G, [&](int g) { return nsplit(g) - 1; });
    for (int g = threadIdx.x; g <= G; g += 256) P.sched[G + 1 + g] = s_pre[g];
  }
  if (P.atomic) {
    const int64_t per = (int64_t)P.M * P.N / 4;
    for (int g = 0; g < G; ++g) {
      if (nsplit(g) < 2) continue;
      f32x4_t* d1 = (f32x4_t*)(P.dw1 + (int64_t)g * P.M * P.N);
      f32x4_t* d2 = (f32x4_t*)(P.dw2 + (int64_t)g * P.M * P.N);
      for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < per; i += (int64_t)gridDim.x * 256) {
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
  const int G = P.groups;
  const int32_t* slot_base = P.sched + (G + 1);
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
template <typename T>
static hipError_t launch_rowgemm_t(const RowGemmParams& P, int kind, int64_t grid, hipStream_t st) {
  switch (kind) {
    case kGemmFc1Fwd:
      rowgemm_kernel<T, false, true, kEpiStore><<<grid, 256, 0, st>>>(P);
      break;
    case kGemmFc2Fwd:
      rowgemm_kernel<T, true, true, kEpiStore><<<grid, 256, 0, st>>>(P);
      break;
    case kGemmFc2Dgrad:
      rowgemm_kernel<T, false, false, kEpiDgrad2><<<grid, 256, 0, st>>>(P);
      break;
    case kGemmFc1Dgrad:
      rowgemm_kernel<T, false, false, kEpiStore><<<grid, 256, 0, st>>>(P);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rowgemm(const RowGemmParams& P, int kind, bool bf16, int64_t grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  return bf16 ? launch_rowgemm_t<uint16_t>(P, kind, grid, st) : launch_rowgemm_t<float>(P, kind, grid, st);
}

hipError_t launch_wgrad(const WgradParams& P, int which, bool bf16, int64_t grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (bf16) {
    if (which == 1)
      wgrad_kernel<uint16_t, true, false, false, false><<<grid, 256, 0, st>>>(P);
    else
      wgrad_kernel<uint16_t, false, true, true, true><<<grid, 256, 0, st>>>(P);
  } else {
    if (which == 1)
      wgrad_kernel<float, true, false, false, false><<<grid, 256, 0, st>>>(P);
    else
      wgrad_kernel<float, false, true, true, true><<<grid, 256, 0, st>>>(P);
  }
  return hipGetLastError();
}

hipError_t launch_wgrad_prep(const WgradPrepParams& P, int64_t grid, hipStream_t st) {
  wgrad_prep_kernel<<<grid, 256, 0, st>>>(P);
  return hipGetLastError();
}

hipError_t launch_wgrad_reduce(const WgradPrepParams& P, int64_t grid, hipStream_t st) {
  wgrad_reduce_kernel<<<grid, 256, 0, st>>>(P);
  return hipGetLastError();
}

int gemm_tile_m(bool bf16) { return bf16 ? Tile<uint16_t>::BM : Tile<float>::BM; }
int gemm_tile_n(bool bf16) { return bf16 ? Tile<uint16_t>::BN : Tile<float>::BN; }

}  // namespace moedet
