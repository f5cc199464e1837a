// Masked dense decode attention: a deliberately plain comparison path (gfx950).
//
// "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding" §4.4
// times one KV window against dense decoding whose attention runs masked,
// fused, or split-K, and shows that a dense baseline which wastes bandwidth
// inflates the window's gain beyond its byte bound.  This file is the masked
// path, written the way a straightforward eager implementation runs it:
//   1. scores S[h, j] = scale * q_h . k_{h/G, j} for every *allocated* row
//      j < cap, rows j >= n_ctx set to -inf (a padding mask); every query
//      head reads its KV head's rows itself (K read G times, no sharing);
//   2. a row softmax of S in place (three passes over each row);
//   3. out_h = sum_j P[h, j] v_{h/G, j} over every allocated row in chunks,
//      the chunks summed in order (V read G times).
// The fused path is the split-K kernel run with one workgroup per query head
// and a single chunk (see attn.hip); the efficient path is split-K proper.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace sd {

constexpr int kNaiveThreads = 256;
constexpr int kScoreRows = 1024;  // rows per score workgroup
constexpr int kPvSplits = 64;     // P.V chunks per query head

template <typename KT, int DH>
__global__ __launch_bounds__(kNaiveThreads) void masked_scores_kernel(
    const float* __restrict__ q, const KT* __restrict__ K, int cap, int n_ctx, int G, float scale,
    float* __restrict__ S) {
  constexpr int LPR = DH / 8;
  constexpr int SLOTS = kNaiveThreads / LPR;
  const int h = blockIdx.y;
  const int sub = threadIdx.x % LPR, slot = threadIdx.x / LPR;
  float qv[8];
  load8f(q + (size_t)h * DH + 8 * sub, qv);
  const KT* Kb = K + (size_t)(h / G) * cap * DH + 8 * sub;
  const int r0 = blockIdx.x * kScoreRows, r1 = min(cap, r0 + kScoreRows);
  for (int j = r0 + slot; j < r1; j += SLOTS) {
    Vec8<KT> kr;
    kr.load(Kb + (size_t)j * DH);
    float kf[8];
    kr.to_float(kf);
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) t = fmaf(kf[e], qv[e], t);
    t = group_sum<LPR>(t);
    if (sub == 0) S[(size_t)h * cap + j] = j < n_ctx ? t * scale : -INFINITY;
  }
}

// P = softmax(S) over each row of cap values, in place; lse[h] = log sum exp(S).
__global__ __launch_bounds__(1024) void masked_softmax_kernel(float* __restrict__ S, int cap,
                                                              float* __restrict__ lse) {
  __shared__ float red[1024 / kWave];
  __shared__ float bcast;
  float* row = S + (size_t)blockIdx.x * cap;
  const int lane = lane_id(), w = threadIdx.x / kWave;
  float m = -INFINITY;
  for (int j = threadIdx.x; j < cap; j += 1024) m = fmaxf(m, row[j]);
  m = wave_max(m);
  if (lane == 0) red[w] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = red[0];
    for (int i = 1; i < 1024 / kWave; ++i) t = fmaxf(t, red[i]);
    bcast = t;
  }
  __syncthreads();
  const float M = bcast;
  float l = 0.f;
  for (int j = threadIdx.x; j < cap; j += 1024) l += __expf(row[j] - M);
  l = wave_sum(l);
  __syncthreads();
  if (lane == 0) red[w] = l;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int i = 0; i < 1024 / kWave; ++i) t += red[i];
    bcast = t;
    if (lse) lse[blockIdx.x] = M + logf(t);
  }
  __syncthreads();
  const float inv = 1.0f / bcast;
  for (int j = threadIdx.x; j < cap; j += 1024) row[j] = __expf(row[j] - M) * inv;
}

// part[h, c, s] partial sums of P[h, j] v_{h/G, j, c} over chunk s of the rows.
template <typename KT, int DH>
__global__ __launch_bounds__(kNaiveThreads) void masked_pv_kernel(
    const float* __restrict__ P, const KT* __restrict__ V, int cap, int n_ctx, int G, int chunk,
    float* __restrict__ part) {
  constexpr int LPR = DH / 8;
  constexpr int SLOTS = kNaiveThreads / LPR;
  __shared__ float red[SLOTS][DH];
  const int s = blockIdx.x, h = blockIdx.y;
  const int sub = threadIdx.x % LPR, slot = threadIdx.x / LPR;
  const KT* Vb = V + (size_t)(h / G) * cap * DH + 8 * sub;
  const float* prow = P + (size_t)h * cap;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  const int r0 = s * chunk, r1 = min(cap, r0 + chunk);
  for (int j = r0 + slot; j < r1; j += SLOTS) {
    Vec8<KT> vr;
    vr.load(Vb + (size_t)j * DH);
    float vf[8];
    vr.to_float(vf);
    const float p = prow[j];  // 0 past n_ctx; rows there are read but may hold anything
    if (j < n_ctx)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(p, vf[e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[slot][8 * sub + e] = acc[e];
  __syncthreads();
  for (int c = threadIdx.x; c < DH; c += kNaiveThreads) {
    float t = 0.f;
    for (int sl = 0; sl < SLOTS; ++sl) t += red[sl][c];
    part[((size_t)h * DH + c) * kPvSplits + s] = t;
  }
}

template <int DH>
__global__ __launch_bounds__(DH) void masked_pv_sum_kernel(const float* __restrict__ part,
                                                           int n_splits, float* __restrict__ out) {
  const int h = blockIdx.x, c = threadIdx.x;
  const float* p = part + ((size_t)h * DH + c) * kPvSplits;
  float t = 0.f;
  for (int s = 0; s < n_splits; ++s) t += p[s];
  out[(size_t)h * DH + c] = t;
}

template <typename KT, int DH>
static void masked_dh(const AttnArgs& a, float* scores, hipStream_t s) {
  const int G = a.h_q / a.h_kv;
  launch_kernel(K_MASKED_SCORES, masked_scores_kernel<KT, DH>,
                dim3((a.cap + kScoreRows - 1) / kScoreRows, a.h_q), dim3(kNaiveThreads), 0, s,
                a.q, (const KT*)a.k, a.cap, a.n_ctx, G, a.scale, scores);
  launch_kernel(K_MASKED_SOFTMAX, masked_softmax_kernel, dim3(a.h_q), dim3(1024), 0, s, scores,
                a.cap, a.lse);
  const int chunk = (a.cap + kPvSplits - 1) / kPvSplits;
  const int n_splits = (a.cap + chunk - 1) / chunk;
  launch_kernel(K_MASKED_PV, masked_pv_kernel<KT, DH>, dim3(n_splits, a.h_q), dim3(kNaiveThreads),
                0, s, (const float*)scores, (const KT*)a.v, a.cap, a.n_ctx, G, chunk, a.pacc);
  launch_kernel(K_MASKED_PV, masked_pv_sum_kernel<DH>, dim3(a.h_q), dim3(DH), 0, s,
                (const float*)a.pacc, n_splits, a.out);
}

void launch_attn_masked(const AttnArgs& a, float* scores, int kv_dtype, hipStream_t s) {
  if (a.dh == 64) {
    if (kv_dtype == 1) masked_dh<bf16_t, 64>(a, scores, s);
    else masked_dh<float, 64>(a, scores, s);
  } else {
    if (kv_dtype == 1) masked_dh<bf16_t, 128>(a, scores, s);
    else masked_dh<float, 128>(a, scores, s);
  }
}

}  // namespace sd
