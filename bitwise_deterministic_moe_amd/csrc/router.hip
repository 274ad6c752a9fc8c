// Router backward: the step directly upstream of dprob ("Trillion-Parameter
// Pretraining Goes Bitwise-Deterministic", section "Interpretation": the
// grouped-GEMM epilogue produces dprob per token and selected expert, and the
// router consumes it).
//
// Router: logits[t, e] = <x_t, wr_e> with weights wr [E, D]; the k largest
// logits are selected and p = softmax over them.  Given dprob [T, k]:
//   dlogits[t, e_j] = p_j * (dprob_j - s_t),  s_t = sum_j p_j dprob_j
//                     (j ascending, float32), 0 for unselected experts;
//   dwr[e, :]       = sum over the routed rows r of expert e, in routing order
//                     (token ascending), of dlogits[t(r), e] * x[t(r), :];
//   dx_router[t, :] = sum over j ascending of dlogits[t, e_j] * wr[e_j, :],
//                     float32 accumulation, one rounding to the storage type.
// dwr is the only reduction across threads.  Deterministic mode sums each
// expert's rows in PH fixed row phases (rows q, q+PH, ... in order) and adds
// the PH phase sums in phase order, with PH = 8 when the mean expert holds
// fewer than 512 rows and d_model is a multiple of 256, else 64 (a function
// of the shapes); the atomic control adds the phase sums into a zeroed dwr
// with atomicAdd, in arrival order.
#include "common.h"
#include "kernels.h"

namespace moedet {

// 8 consecutive elements of the storage type as floats (16 bytes for bf16,
// 32 for float32); p must be 16-byte aligned.
DEV void load8(const uint16_t* p, float (&f)[8]) {
  const u32x4_t v = *(const u32x4_t*)p;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f[2 * w] = bf16_to_f32(v[w] & 0xffffu);
    f[2 * w + 1] = bf16_to_f32(v[w] >> 16);
  }
}
DEV void load8(const float* p, float (&f)[8]) {
  const f32x4_t a = *(const f32x4_t*)p, b = *(const f32x4_t*)(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = a[i];
    f[4 + i] = b[i];
  }
}
DEV void store8(uint16_t* p, const float (&f)[8]) {
  u32x4_t v;
#pragma unroll
  for (int w = 0; w < 4; ++w) v[w] = pack_bf16x2(f[2 * w], f[2 * w + 1]);
  *(u32x4_t*)p = v;
}
DEV void store8(float* p, const float (&f)[8]) {
  *(f32x4_t*)p = f32x4_t{f[0], f[1], f[2], f[3]};
  *(f32x4_t*)(p + 4) = f32x4_t{f[4], f[5], f[6], f[7]};
}

// One wave per token (4 tokens per workgroup): lane j < k holds slot j; the
// sum s is taken in slot order by every lane.  The dense row is built in LDS
// (zeros, then the k values) and copied out with coalesced stores, so every
// element of dlogits is written once.
__global__ __launch_bounds__(256) void router_dlogits_kernel(RouterParams P) {
  __shared__ float s_row[4][kMaxExperts];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t units = (P.T + 3) / 4;
  const int64_t u = map_unit(blockIdx.x, units, P.seed);
  const int64_t t = u * 4 + wave;
  const bool live = u >= 0 && t < P.T;
  float prod = 0.f, p = 0.f, g = 0.f;
  int32_t e = -1;
  if (live && lane < P.k) {
    p = P.topk_prob[t * P.k + lane];
    g = P.dprob[t * P.k + lane];
    e = P.topk_idx[t * P.k + lane];
    prod = p * g;
  }
  float s = 0.f;
  for (int i = 0; i < P.k; ++i) s = s + __shfl(prod, i);
  for (int c = lane; c < P.E; c += kWave) s_row[wave][c] = 0.f;
  __syncthreads();
  if (live && lane < P.k) s_row[wave][e] = p * (g - s);
  __syncthreads();
  if (!live) return;
  float* row = P.dlogits + t * P.E;
  for (int c = lane; c < P.E; c += kWave) row[c] = s_row[wave][c];
}

// dwr[e, d0 .. d0 + 8*LN - 1] with PH row phases and LN = 256 / PH lanes:
// thread (q, c) = (tid / LN, tid % LN) sums 8 columns d0 + 8c .. +7 over the
// expert's rows q, q+PH, q+2PH, ... (routing order), four rows per step so
// that their loads are in flight together; the PH phase sums are then added in
// phase order.  PH is a function of the shapes only (more phases when the
// experts hold many rows).
template <typename T, int PH>
__global__ __launch_bounds__(256) void router_dwr_kernel(RouterParams P) {
  constexpr int LN = 256 / PH, W = 8 * LN;
  __shared__ float s_part[PH][W + 1];
  const int nd = P.D / W;
  const int64_t u = map_unit(blockIdx.x, (int64_t)P.E * nd, P.seed);
  if (u < 0) return;
  const int e = (int)(u / nd), d0 = (int)(u % nd) * W;
  const int q = threadIdx.x / LN, c = threadIdx.x % LN;
  const int64_t r0 = P.offsets[e], cnt = P.counts[e];
  const T* x = (const T*)P.x + d0 + 8 * c;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int64_t r = q; r < cnt; r += 4 * PH) {
    int64_t t[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) t[b] = r + b * PH < cnt ? P.row_tok[r0 + r + b * PH] : -1;
    float dl[4], f[4][8];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      dl[b] = t[b] >= 0 ? P.dlogits[t[b] * P.E + e] : 0.f;
      load8(x + (t[b] >= 0 ? t[b] : 0) * P.D, f[b]);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (t[b] >= 0)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(dl[b], f[b][i], acc[i]);
  }
  float* out = P.dwr + (int64_t)e * P.D + d0;
  if (P.atomic) {
    if (cnt > q)
#pragma unroll
      for (int i = 0; i < 8; ++i) atomicAdd(out + 8 * c + i, acc[i]);
    return;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) s_part[q][8 * c + i] = acc[i];
  __syncthreads();
  if (threadIdx.x < W) {
    float v = s_part[0][threadIdx.x];
    for (int qq = 1; qq < PH; ++qq) v = v + s_part[qq][threadIdx.x];
    out[threadIdx.x] = v;
  }
}

// dx_router[t, d .. d+7] = sum_j dlogits[t, e_j] * wr[e_j, d .. d+7], j
// ascending, the selected experts taken eight at a time so that their loads
// are in flight together.
template <typename T>
__global__ __launch_bounds__(256) void router_dx_kernel(RouterParams P) {
  const int per = P.D / 8;
  const int64_t units = (P.T * per + 255) / 256;
  const int64_t u = map_unit(blockIdx.x, units, P.seed);
  if (u < 0) return;
  const int64_t idx = u * 256 + threadIdx.x;
  if (idx >= P.T * per) return;
  const int64_t t = idx / per;
  const int d = (int)(idx % per) * 8;
  const T* wr = (const T*)P.wr + d;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int j0 = 0; j0 < P.k; j0 += 8) {
    int e[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) e[b] = j0 + b < P.k ? P.topk_idx[t * P.k + j0 + b] : -1;
    float dl[8], f[8][8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      dl[b] = e[b] >= 0 ? P.dlogits[t * P.E + e[b]] : 0.f;
      load8(wr + (int64_t)(e[b] >= 0 ? e[b] : 0) * P.D, f[b]);
    }
#pragma unroll
    for (int b = 0; b < 8; ++b)
      if (e[b] >= 0)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(dl[b], f[b][i], acc[i]);
  }
  store8((T*)P.dx + t * P.D + d, acc);
}

hipError_t launch_router_bwd(const RouterParams& P, bool bf16, hipStream_t st) {
  if (P.T > 0) {
    router_dlogits_kernel<<<grid_for_units((P.T + 3) / 4), 256, 0, st>>>(P);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (P.atomic) {
    hipError_t e = launch_zero(P.dwr, (int64_t)P.E * P.D, st);
    if (e != hipSuccess) return e;
  }
  const int W = 8 * (256 / P.phases);
  const int64_t g2 = grid_for_units((int64_t)P.E * (P.D / W));
  if (P.phases == 8) {
    if (bf16)
      router_dwr_kernel<uint16_t, 8><<<g2, 256, 0, st>>>(P);
    else
      router_dwr_kernel<float, 8><<<g2, 256, 0, st>>>(P);
  } else {
    if (bf16)
      router_dwr_kernel<uint16_t, 64><<<g2, 256, 0, st>>>(P);
    else
      router_dwr_kernel<float, 64><<<g2, 256, 0, st>>>(P);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || P.T == 0) return e;
  const int64_t g3 = grid_for_units((P.T * (P.D / 8) + 255) / 256);
  if (bf16)
    router_dx_kernel<uint16_t><<<g3, 256, 0, st>>>(P);
  else
    router_dx_kernel<float><<<g3, 256, 0, st>>>(P);
  return hipGetLastError();
}

}  // namespace moedet
