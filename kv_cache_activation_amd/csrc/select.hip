// One-time attention-scored KV selection (gfx950, wave64).
//
// "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding"
// §4.1: after prefill the cache is scored once with the attention of an
// observation window of queries; sinks, the window and the best-scoring rows
// of each KV head are kept and gathered into a contiguous buffer.
//
// Kernels, in launch order:
//   lse_partial  grid (key chunks, KV heads); one key row per thread held in
//                VGPRs, window queries staged in LDS in batches of 32.  For each
//                query: the causal logits of the chunk's keys, a wave max/sum
//                and a four-wave merge -> partial (max, sum) per (chunk, query).
//   lse_final    one thread per window query: merge the chunk partials into
//                the query's log-sum-exp (log2 domain).
//   score        same layout as lse_partial; each thread sums, over the G*w
//                queries of its KV head in a fixed order, the softmax weight
//                that the query puts on its key -> scores[kv, j].
//   topk         one 1024-thread workgroup per KV head: an 8-bit-digit radix
//                select on order-preserving keys of the float32 scores finds
//                the m-th largest candidate value T; each wave then counts its
//                contiguous range with ballots, two block scans place the
//                ranges, and each wave emits, in ascending position, the
//                sinks, the window, all candidates above T and the
//                lowest-position candidates equal to T up to m (ties to the
//                lower position).
//   gather       16-byte copies of the kept K and V rows into the buffer.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace sd {

constexpr int kSelThreads = 256;  // == key chunk length
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kQBatch = 32;
constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;

template <typename KT, int DH>
__device__ __forceinline__ void load_row_f32(const KT* p, float (&r)[DH]) {
#pragma unroll
  for (int c = 0; c < DH; c += 8) {
    Vec8<KT> v;
    v.load_cached(p + c);
    float f[8];
    v.to_float(f);
#pragma unroll
    for (int e = 0; e < 8; ++e) r[c + e] = f[e];
  }
}

template <int DH>
__device__ __forceinline__ float dot_lds(const float (&r)[DH], const float* qs) {
  float a = 0.f;
#pragma unroll
  for (int c = 0; c < DH; c += 4) {
    const float4 qq = *reinterpret_cast<const float4*>(qs + c);
    a = fmaf(r[c], qq.x, a);
    a = fmaf(r[c + 1], qq.y, a);
    a = fmaf(r[c + 2], qq.z, a);
    a = fmaf(r[c + 3], qq.w, a);
  }
  return a;
}

// Stage window queries qb..qb+kQBatch-1 of KV head kv into LDS.  Query index
// qi = g * w + i is head kv*G + g at window slot i.
template <int DH>
__device__ void stage_queries(const float* __restrict__ q_win, int kv, int G, int w, int qb,
                              int Q, float (*qs)[DH]) {
  for (int t = threadIdx.x; t < kQBatch * DH; t += blockDim.x) {
    const int qq = t / DH, c = t - qq * DH;
    const int qi = qb + qq;
    float v = 0.f;
    if (qi < Q) {
      const int g = qi / w, i = qi - g * w;
      v = q_win[((size_t)(kv * G + g) * w + i) * DH + c];
    }
    qs[qq][c] = v;
  }
}

template <typename KT, int DH>
__global__ __launch_bounds__(kSelThreads) void sel_lse_partial_kernel(
    const KT* __restrict__ K, int cap, int n, const float* __restrict__ q_win, int w, int G,
    float scale_log2, int n_chunks, float* __restrict__ lse_part) {
  __shared__ float qs[kQBatch][DH];
  __shared__ float red_m[kSelWaves][kQBatch], red_l[kSelWaves][kQBatch];
  const int chunk = blockIdx.x, kv = blockIdx.y;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int j = chunk * kSelThreads + threadIdx.x;
  const bool have = j < n;
  float kr[DH];
  if (have) {
    load_row_f32<KT, DH>(K + ((size_t)kv * cap + j) * DH, kr);
  } else {
#pragma unroll
    for (int c = 0; c < DH; ++c) kr[c] = 0.f;
  }
  const int Q = G * w;
  for (int qb = 0; qb < Q; qb += kQBatch) {
    __syncthreads();
    stage_queries<DH>(q_win, kv, G, w, qb, Q, qs);
    __syncthreads();
    for (int qq = 0; qq < kQBatch && qb + qq < Q; ++qq) {
      const int i = (qb + qq) % w;
      const bool vis = have && j <= n - w + i;
      const float z = vis ? dot_lds<DH>(kr, qs[qq]) * scale_log2 : -INFINITY;
      const float mw = wave_max(z);
      const float e = vis ? exp2f(z - mw) : 0.f;
      const float lw = wave_sum(e);
      if (lane == 0) {
        red_m[wave][qq] = mw;
        red_l[wave][qq] = lw;
      }
    }
    __syncthreads();
    if (threadIdx.x < kQBatch && qb + threadIdx.x < Q) {
      const int qq = threadIdx.x;
      float M = -INFINITY;
#pragma unroll
      for (int v = 0; v < kSelWaves; ++v) M = fmaxf(M, red_m[v][qq]);
      float L = 0.f;
#pragma unroll
      for (int v = 0; v < kSelWaves; ++v)
        if (red_m[v][qq] != -INFINITY) L = fmaf(red_l[v][qq], exp2f(red_m[v][qq] - M), L);
      float* o = lse_part + (((size_t)kv * n_chunks + chunk) * Q + qb + qq) * 2;
      o[0] = M;
      o[1] = L;
    }
  }
}

// One wave per window query: lane l merges chunks l, l + 64, ... (all of its
// loads issued together), then a wave max and a wave sum in a fixed order.
constexpr int kLsePer = 32;  // chunks per lane in one pass (n_chunks <= 64 * 32 per pass)
__global__ __launch_bounds__(256) void sel_lse_final_kernel(const float* __restrict__ lse_part,
                                                            int n_chunks, int G, int w, int h_kv,
                                                            float* __restrict__ lse) {
  const int Q = G * w;
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;  // query of the wave
  if (t >= h_kv * Q) return;  // wave-uniform
  const int lane = lane_id();
  const int kv = t / Q, qi = t - kv * Q;
  const float2* p = reinterpret_cast<const float2*>(lse_part) + (size_t)kv * n_chunks * Q + qi;
  float M = -INFINITY, L = 0.f;
  for (int c0 = 0; c0 < n_chunks; c0 += kWave * kLsePer) {
    float2 v[kLsePer];
#pragma unroll
    for (int u = 0; u < kLsePer; ++u) {
      const int c = min(c0 + lane + kWave * u, n_chunks - 1);
      v[u] = p[(size_t)c * Q];
    }
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < kLsePer; ++u)
      if (c0 + lane + kWave * u < n_chunks) m = fmaxf(m, v[u].x);
    const float mn = fmaxf(M, m);
    float l = 0.f;
#pragma unroll
    for (int u = 0; u < kLsePer; ++u)
      if (c0 + lane + kWave * u < n_chunks && v[u].x != -INFINITY)
        l = fmaf(v[u].y, exp2f(v[u].x - mn), l);
    L = (M == -INFINITY ? 0.f : L * exp2f(M - mn)) + l;
    M = mn;
  }
  const float MW = wave_max(M);
  const float LW = wave_sum(M == -INFINITY ? 0.f : L * exp2f(M - MW));
  if (lane == 0) {
    const int g = qi / w, i = qi - g * w;
    lse[(kv * G + g) * w + i] = MW + log2f(LW);
  }
}

template <typename KT, int DH>
__global__ __launch_bounds__(kSelThreads) void sel_score_kernel(
    const KT* __restrict__ K, int cap, int n, const float* __restrict__ q_win, int w, int G,
    float scale_log2, const float* __restrict__ lse, float* __restrict__ scores) {
  __shared__ float qs[kQBatch][DH];
  __shared__ float ls[kQBatch];
  const int chunk = blockIdx.x, kv = blockIdx.y;
  const int j = chunk * kSelThreads + threadIdx.x;
  const bool have = j < n;
  float kr[DH];
  if (have) {
    load_row_f32<KT, DH>(K + ((size_t)kv * cap + j) * DH, kr);
  } else {
#pragma unroll
    for (int c = 0; c < DH; ++c) kr[c] = 0.f;
  }
  const int Q = G * w;
  float s = 0.f;
  for (int qb = 0; qb < Q; qb += kQBatch) {
    __syncthreads();
    stage_queries<DH>(q_win, kv, G, w, qb, Q, qs);
    if (threadIdx.x < kQBatch) {
      const int qi = qb + threadIdx.x;
      float v = 0.f;
      if (qi < Q) {
        const int g = qi / w, i = qi - g * w;
        v = lse[(kv * G + g) * w + i];
      }
      ls[threadIdx.x] = v;
    }
    __syncthreads();
    for (int qq = 0; qq < kQBatch && qb + qq < Q; ++qq) {
      const int i = (qb + qq) % w;
      if (have && j <= n - w + i) s += exp2f(dot_lds<DH>(kr, qs[qq]) * scale_log2 - ls[qq]);
    }
  }
  if (have) scores[(size_t)kv * n + j] = s;
}

// ------------------------------------------------------------------ matrix cores
// Scoring with bf16 caches on the matrix cores.  Per KV head the logits are a
// product Z [G w, n] = Q_win [G w, d_h] K^T [d_h, n] with d_h-long dot
// products: about 2 G w flops per cache byte, a dense contraction, so
// v_mfma_f32_16x16x32_bf16 computes them.  The window queries are float32:
// each is split into three bf16 parts (hi + mid + lo carries its 24-bit
// significand), the bf16 keys are exact, every product is exact in float32 and
// the sums accumulate in float32, so the logits have float32 accuracy, as on
// the vector ALUs.  Operand layout (lane l): A = queries, row l % 16, dims
// 8 (l / 16) + e of each 32-dim step; B = keys, column l % 16 (one key row,
// 16 contiguous bytes per lane and step); result rows 4 (l / 16) + r, column
// l % 16.
//   A workgroup (four waves) takes a chunk of 256 keys of one KV head, each
//   wave 64 of them (four 16-key tiles) held in registers; the queries go
//   through LDS in batches of 64 (four 16-query tiles).  lse pass: each query's (max, sum of 2^z) over the wave's visible
//   keys (DPP over the 16 lanes of a result row), then over the four waves in
//   LDS -> the chunk partial, as the vector-ALU kernel writes it.  score pass:
//   each key's sum over the queries of 2^(z - lse), lanes of one column added
//   with lane swaps, accumulated over the query tiles in a fixed order.
constexpr int kSelQB = 64;  // queries staged per batch (four 16-row tiles)
constexpr int kSelSub = 1;  // key chunks per workgroup (measured: staging once for 2 or 4
                            // chunks, or batches of 128 queries, were no faster)

// Staged queries on the matrix-core path: the three bf16 parts (hi, mid, lo)
// of kSelQB query rows, part p of row r at qp[(p kSelQB + r) QS + dim], rows
// padded to QS = DH + 8 elements (16-byte aligned rows, reads spread over the
// LDS banks).
template <int DH>
constexpr int sel_qs() { return DH + 8; }

// Logits of one 16-query tile (staged rows from qrow) against the wave's four
// 16-key tiles: z[c][r] for query 4 (l / 16) + r of the tile and key column
// l % 16 of key tile c.  The A operands are the staged parts, read as is.
template <int DH>
__device__ __forceinline__ void sel_tile_logits(const bf16_t* qp, int qrow,
                                                const u32x4 (&kf)[4][DH / 32], f32x4 (&z)[4]) {
  constexpr int NS = DH / 32, QS = sel_qs<DH>();
  const int lane = lane_id();
#pragma unroll
  for (int c = 0; c < 4; ++c) z[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const bf16_t* base = qp + (qrow + lane % 16) * QS + 32 * st + 8 * (lane / 16);
    const u32x4 ah = *reinterpret_cast<const u32x4*>(base);
    const u32x4 am = *reinterpret_cast<const u32x4*>(base + kSelQB * QS);
    const u32x4 al = *reinterpret_cast<const u32x4*>(base + 2 * kSelQB * QS);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      z[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah), as_bf16x8(kf[c][st]),
                                                     z[c], 0, 0, 0);
      z[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(am), as_bf16x8(kf[c][st]),
                                                     z[c], 0, 0, 0);
      z[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(al), as_bf16x8(kf[c][st]),
                                                     z[c], 0, 0, 0);
    }
  }
}

// Keys of the wave: four tiles of 16 from key j0, 16 bytes per lane and step
// (rows past n read row n - 1 and are masked by the callers).
template <int DH>
__device__ __forceinline__ void sel_load_keys(const bf16_t* __restrict__ Kh, int n, int j0,
                                              u32x4 (&kf)[4][DH / 32]) {
  const int lane = lane_id();
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int j = min(j0 + 16 * c + lane % 16, n - 1);
#pragma unroll
    for (int st = 0; st < DH / 32; ++st)
      kf[c][st] = *reinterpret_cast<const u32x4*>(Kh + (size_t)j * DH + 32 * st + 8 * (lane / 16));
  }
}

// Stage queries [qb, qb + kSelQB) of KV head kv as their three bf16 parts
// (split once per staging, not once per key chunk and wave).
template <int DH>
__device__ void sel_stage_q(const float* __restrict__ q_win, int kv, int Q, int qb, bf16_t* qp) {
  constexpr int QS = sel_qs<DH>();
  const float* src = q_win + (size_t)kv * Q * DH;
  for (int t = threadIdx.x; t < kSelQB * DH / 8; t += kSelThreads) {
    const int qq = t / (DH / 8), c8 = t - qq * (DH / 8);
    float xv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (qb + qq < Q) load8f(src + (size_t)(qb + qq) * DH + 8 * c8, xv);
    u32x4 hi, mid, lo;
    split3_bf16(xv, hi, mid, lo);
    bf16_t* dst = qp + qq * QS + 8 * c8;
    *reinterpret_cast<u32x4*>(dst) = hi;
    *reinterpret_cast<u32x4*>(dst + kSelQB * QS) = mid;
    *reinterpret_cast<u32x4*>(dst + 2 * kSelQB * QS) = lo;
  }
}

// Raw v_exp_f32 (2^x, -inf -> 0); its arguments here are at most 0.
__device__ __forceinline__ float sel_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int DH>
__global__ __launch_bounds__(kSelThreads) void sel_lse_partial_mfma_kernel(
    const bf16_t* __restrict__ K, int cap, int n, const float* __restrict__ q_win, int w, int G,
    float scale_log2, int n_chunks, float* __restrict__ lse_part) {
  __shared__ __align__(16) bf16_t qs[3 * kSelQB * sel_qs<DH>()];
  __shared__ float red_m[kSelWaves][kSelQB], red_l[kSelWaves][kSelQB];
  const int kv = blockIdx.y;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int Q = G * w;
#pragma unroll 1
  for (int sub = 0; sub < kSelSub; ++sub) {
    const int chunk = blockIdx.x * kSelSub + sub;
    if (chunk >= n_chunks) break;  // workgroup-uniform
    const int j0 = chunk * kSelThreads + wave * 64;
    // the chunk's keys once, for every query batch
    u32x4 kf[4][DH / 32];
    sel_load_keys<DH>(K + (size_t)kv * cap * DH, n, j0, kf);
  for (int qb = 0; qb < Q; qb += kSelQB) {
    __syncthreads();
    sel_stage_q<DH>(q_win, kv, Q, qb, qs);
    __syncthreads();
#pragma unroll 1
    for (int rt = 0; rt < kSelQB / 16; ++rt) {
      f32x4 z[4];
      sel_tile_logits<DH>(qs, 16 * rt, kf, z);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ql = 16 * rt + 4 * (lane / 16) + r, q = qb + ql;
        const int i = q % w;
        float zz[4], mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = j0 + 16 * c + lane % 16;
          const bool vis = q < Q && j < n && j <= n - w + i;
          zz[c] = vis ? z[c][r] * scale_log2 : -INFINITY;
          mx = fmaxf(mx, zz[c]);
        }
        mx = group_max<16>(mx);
        float e = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) e += zz[c] == -INFINITY ? 0.f : sel_exp2(zz[c] - mx);
        e = group_sum<16>(e);
        if (lane % 16 == 0) {
          red_m[wave][ql] = mx;
          red_l[wave][ql] = e;
        }
      }
    }
    __syncthreads();
    if (threadIdx.x < kSelQB && qb + threadIdx.x < Q) {
      const int ql = threadIdx.x;
      float M = -INFINITY;
#pragma unroll
      for (int v = 0; v < kSelWaves; ++v) M = fmaxf(M, red_m[v][ql]);
      float L = 0.f;
#pragma unroll
      for (int v = 0; v < kSelWaves; ++v)
        if (red_m[v][ql] != -INFINITY) L = fmaf(red_l[v][ql], sel_exp2(red_m[v][ql] - M), L);
      float* o = lse_part + (((size_t)kv * n_chunks + chunk) * Q + qb + ql) * 2;
      o[0] = M;
      o[1] = L;
    }
    __syncthreads();  // red_m / red_l are reused by the next query batch
  }
  }
}

template <int DH>
__global__ __launch_bounds__(kSelThreads) void sel_score_mfma_kernel(
    const bf16_t* __restrict__ K, int cap, int n, const float* __restrict__ q_win, int w, int G,
    float scale_log2, const float* __restrict__ lse, float* __restrict__ scores) {
  __shared__ __align__(16) bf16_t qs[3 * kSelQB * sel_qs<DH>()];
  __shared__ float ls[kSelQB];
  const int kv = blockIdx.y;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int Q = G * w;
#pragma unroll 1
  for (int sub = 0; sub < kSelSub; ++sub) {
  const int chunk = blockIdx.x * kSelSub + sub;
  if (chunk * kSelThreads >= n) break;  // workgroup-uniform
  const int j0 = chunk * kSelThreads + wave * 64;
  u32x4 kf[4][DH / 32];
  sel_load_keys<DH>(K + (size_t)kv * cap * DH, n, j0, kf);
  float sc[4] = {0.f, 0.f, 0.f, 0.f};  // per key tile, this lane's column
  for (int qb = 0; qb < Q; qb += kSelQB) {
    if (sub == 0 || Q > kSelQB) {  // one batch: staged once for all chunks
      __syncthreads();
      sel_stage_q<DH>(q_win, kv, Q, qb, qs);
      if (threadIdx.x < kSelQB)  // lse of query q = g w + i is lse[(kv G + g) w + i]
        ls[threadIdx.x] = qb + threadIdx.x < Q ? lse[(size_t)kv * Q + qb + threadIdx.x] : 0.f;
      __syncthreads();
    }
#pragma unroll 1
    for (int rt = 0; rt < kSelQB / 16; ++rt) {
      f32x4 z[4];
      sel_tile_logits<DH>(qs, 16 * rt, kf, z);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = j0 + 16 * c + lane % 16;
        float part = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ql = 16 * rt + 4 * (lane / 16) + r, q = qb + ql;
          const bool vis = q < Q && j < n && j <= n - w + q % w;
          part += vis ? sel_exp2(z[c][r] * scale_log2 - ls[ql]) : 0.f;
        }
        // add the four row groups of the column (lanes l, l ^ 16, l ^ 32, l ^ 48)
        part += xor_lanes<16>(part);
        part += xor_lanes<32>(part);
        sc[c] += part;
      }
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = j0 + 16 * c + lane;
      if (j < n) scores[(size_t)kv * n + j] = sc[c];
    }
  }
  }
}

// Order-preserving map of float32 to uint32 (larger float -> larger key);
// -0 and +0 map to one key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = f == 0.f ? 0u : __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-wide exclusive prefix sum of per-thread counts (thread order), plus
// the block total: a DPP wave scan, then the wave totals through LDS.
__device__ __forceinline__ int block_excl_sum(int x, int* wave_tot, int& total) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int incl = wave_incl_scan(x);
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
  for (int v = 0; v < kTopkWaves; ++v) {
    if (v < wave) before += wave_tot[v];
    total += wave_tot[v];
  }
  __syncthreads();
  return before + incl - x;
}

__global__ __launch_bounds__(kTopkThreads) void sel_topk_kernel(const float* __restrict__ scores,
                                                                 int n, int w, int n_sink,
                                                                 int k_keep_all, int ragged,
                                                                 HeadInts k_heads, int stride,
                                                                 int32_t* __restrict__ idx) {
  __shared__ unsigned hist[256];
  __shared__ unsigned sh_prefix, sh_need;
  __shared__ int wave_tot[kTopkWaves];
  const int kv = blockIdx.x;
  const float* S = scores + (size_t)kv * n;
  // this head's budget (one budget for all heads unless ragged)
  const int k_keep = ragged ? k_heads.v[kv & (kMaxKvHeads - 1)] : k_keep_all;
  int32_t* out = idx + (size_t)kv * stride;
  if (k_keep >= n) {
    for (int j = threadIdx.x; j < n; j += kTopkThreads) out[j] = j;
    return;
  }
  const int m = k_keep - n_sink - w;
  const int c0 = n_sink, c1 = n - w;
  unsigned T = 0, need = 0;
  if (m > 0) {
    // the m-th largest candidate key T: four 8-bit digit passes, each a
    // histogram of the candidates whose higher digits match those found
    unsigned prefix = 0;
    need = (unsigned)m;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int bb = threadIdx.x; bb < 256; bb += kTopkThreads) hist[bb] = 0u;
      __syncthreads();
      // eight scores per thread in flight (from clamped, always valid
      // positions) before their histogram adds
      constexpr int HU = 8;
      for (int j0 = c0; j0 < c1; j0 += kTopkThreads * HU) {  // uniform trip count
        unsigned key[HU];
#pragma unroll
        for (int u = 0; u < HU; ++u)
          key[u] = order_key(S[min(j0 + (int)threadIdx.x + kTopkThreads * u, c1 - 1)]);
#pragma unroll
        for (int u = 0; u < HU; ++u) {
          const int j = j0 + (int)threadIdx.x + kTopkThreads * u;
          const bool match =
              j < c1 && (pass == 0 || (key[u] >> (shift + 8)) == (prefix >> (shift + 8)));
          if (match) atomicAdd(&hist[(key[u] >> shift) & 255u], 1u);
        }
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        unsigned above = 0;
        int bb = 255;
        for (; bb > 0; --bb) {
          if (above + hist[bb] >= need) break;
          above += hist[bb];
        }
        sh_prefix = prefix | ((unsigned)bb << shift);
        sh_need = need - above;
      }
      __syncthreads();
      prefix = sh_prefix;
      need = sh_need;
      __syncthreads();
    }
    T = prefix;
  }
  // emission in ascending position: wave v owns positions [v R, v R + R),
  // read 64 at a time (coalesced); kept are the forced rows, candidates above
  // T, and the first `need` candidates equal to T in position order.  A
  // first sweep counts, two block scans place the waves, a second sweep
  // writes with ballot ranks.
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int R = (n + kTopkWaves - 1) / kTopkWaves;
  const int p0 = min(n, wave * R), p1 = min(n, p0 + R);
  // eight 64-position blocks per step, their loads in flight together
  constexpr int EU = 8;
  auto key_at = [&](int j) { return order_key(S[min(j, n - 1)]); };
  int n_take = 0, n_eq = 0;  // wave totals (uniform)
  for (int jb = p0; jb < p1; jb += kWave * EU) {
    unsigned kk[EU];
#pragma unroll
    for (int u = 0; u < EU; ++u) kk[u] = key_at(jb + kWave * u + lane);
#pragma unroll
    for (int u = 0; u < EU; ++u) {
      const int j = jb + kWave * u + lane;
      const bool valid = j < p1;
      const bool forced = valid && (j < c0 || j >= c1);
      const bool cand = valid && !forced && m > 0;
      n_take += __popcll(__ballot(forced || (cand && kk[u] > T)));
      n_eq += __popcll(__ballot(cand && kk[u] == T));
    }
  }
  int eq_total;
  const int eq_before = block_excl_sum(lane == 0 ? n_eq : 0, wave_tot, eq_total);
  const int eq_wave = __shfl(eq_before, 0);
  const int ties = max(0, min(n_eq, (int)need - eq_wave));  // ties this wave keeps
  int take_total;
  const int pos_before = block_excl_sum(lane == 0 ? n_take + ties : 0, wave_tot, take_total);
  int pos = __shfl(pos_before, 0), eq_seen = 0;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int jb = p0; jb < p1; jb += kWave * EU) {
    unsigned kk[EU];
#pragma unroll
    for (int u = 0; u < EU; ++u) kk[u] = key_at(jb + kWave * u + lane);
#pragma unroll
    for (int u = 0; u < EU; ++u) {
      const int j = jb + kWave * u + lane;
      const bool valid = j < p1;
      const bool forced = valid && (j < c0 || j >= c1);
      const bool cand = valid && !forced && m > 0;
      const bool eq = cand && kk[u] == T;
      const unsigned long long eqm = __ballot(eq);
      const bool take = forced || (cand && kk[u] > T) ||
                        (eq && eq_seen + __popcll(eqm & below) < ties);
      const unsigned long long tm = __ballot(take);
      if (take) {
        const int p = pos + __popcll(tm & below);
        if (p < k_keep) out[p] = j;  // p < k_keep always; guard anyway
      }
      pos += __popcll(tm);
      eq_seen += __popcll(eqm);
    }
  }
}

template <typename KT, int DH>
__global__ void sel_gather_kernel(const KT* __restrict__ K, const KT* __restrict__ V,
                                  int cap_full, const int32_t* __restrict__ idx, int k_eff_all,
                                  int ragged, HeadInts k_eff_heads, int stride,
                                  KT* __restrict__ Ks, KT* __restrict__ Vs, int cap_sel) {
  constexpr int P = DH * (int)sizeof(KT) / 16;  // 16-byte pieces per row
  const int kv = blockIdx.y;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int r = t / P, piece = t - r * P;
  const int k_eff = ragged ? k_eff_heads.v[kv & (kMaxKvHeads - 1)] : k_eff_all;
  if (r >= k_eff) return;
  const int src = idx[(size_t)kv * stride + r];
  if (src < 0 || src >= cap_full) return;  // indices come from data: never read outside
  const uint4* ks = reinterpret_cast<const uint4*>(K + ((size_t)kv * cap_full + src) * DH) + piece;
  const uint4* vs = reinterpret_cast<const uint4*>(V + ((size_t)kv * cap_full + src) * DH) + piece;
  uint4* kd = reinterpret_cast<uint4*>(Ks + ((size_t)kv * cap_sel + r) * DH) + piece;
  uint4* vd = reinterpret_cast<uint4*>(Vs + ((size_t)kv * cap_sel + r) * DH) + piece;
  *kd = *ks;
  *vd = *vs;
}

// ------------------------------------------------------------------ chunked top-k
// The same selection (m largest candidate keys, ties to the lower position,
// ascending list with the forced rows) spread over C chunks of kTopkChunk
// positions per KV head, for long contexts where one workgroup per head
// leaves the chip nearly idle.  Four digit passes, each a chunk histogram
// launch and a per-head pick launch (state[kv] = (prefix, need)); then each
// chunk counts what it keeps, and each chunk emits its part of the list at
// the offset that the counts of the chunks before it give (ties go to the
// first `need` equal candidates in position order, chunk by chunk).
constexpr int kTopkChunk = 4096;

__device__ __forceinline__ int topk_budget(int ragged, const HeadInts& k_heads, int k_keep_all,
                                           int kv) {
  return ragged ? k_heads.v[kv & (kMaxKvHeads - 1)] : k_keep_all;
}

__global__ __launch_bounds__(kTopkThreads) void sel_topk_hist_kernel(
    const float* __restrict__ scores, int n, int w, int n_sink, int k_keep_all, int ragged,
    HeadInts k_heads, int pass, const unsigned* __restrict__ state, unsigned* __restrict__ hist) {
  __shared__ unsigned h[256];
  const int ch = blockIdx.x, kv = blockIdx.y, C = gridDim.x;
  const float* S = scores + (size_t)kv * n;
  const int k_keep = topk_budget(ragged, k_heads, k_keep_all, kv);
  const int m = k_keep - n_sink - w;
  for (int b = threadIdx.x; b < 256; b += kTopkThreads) h[b] = 0u;
  __syncthreads();
  if (k_keep < n && m > 0) {  // workgroup-uniform
    const int shift = 24 - 8 * pass;
    const unsigned prefix = pass ? state[2 * kv] : 0u;
    const int c0 = max(n_sink, ch * kTopkChunk), c1 = min(n - w, (ch + 1) * kTopkChunk);
    constexpr int HU = kTopkChunk / kTopkThreads;  // keys per thread, all in flight
    if (c0 < c1) {
      unsigned key[HU];
#pragma unroll
      for (int u = 0; u < HU; ++u)
        key[u] = order_key(S[min(c0 + (int)threadIdx.x + kTopkThreads * u, c1 - 1)]);
#pragma unroll
      for (int u = 0; u < HU; ++u) {
        const int j = c0 + (int)threadIdx.x + kTopkThreads * u;
        const bool match =
            j < c1 && (pass == 0 || (key[u] >> (shift + 8)) == (prefix >> (shift + 8)));
        if (match) atomicAdd(&h[(key[u] >> shift) & 255u], 1u);
      }
    }
  }
  __syncthreads();
  unsigned* out = hist + ((size_t)kv * C + ch) * 256;
  for (int b = threadIdx.x; b < 256; b += kTopkThreads) out[b] = h[b];
}

__global__ __launch_bounds__(256) void sel_topk_pick_kernel(int n, int w, int n_sink,
                                                            int k_keep_all, int ragged,
                                                            HeadInts k_heads, int pass, int C,
                                                            unsigned* __restrict__ state,
                                                            const unsigned* __restrict__ hist) {
  __shared__ unsigned binv[256], sfx[257], wave_sum_s[4];
  const int kv = blockIdx.x, t = threadIdx.x, lane = lane_id(), wave = threadIdx.x / kWave;
  const int k_keep = topk_budget(ragged, k_heads, k_keep_all, kv);
  const int m = k_keep - n_sink - w;
  if (k_keep >= n || m <= 0) return;  // workgroup-uniform; the count kernel does not read state
  // bin t's total over the chunks, eight loads in flight at a time
  const unsigned* hb = hist + (size_t)kv * C * 256 + t;
  unsigned part[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  for (int c0 = 0; c0 < C; c0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (c0 + u < C) part[u] += hb[(size_t)(c0 + u) * 256];
  }
  unsigned tot = 0u;
#pragma unroll
  for (int u = 0; u < 8; ++u) tot += part[u];
  binv[t] = tot;
  __syncthreads();
  // suffix sums: thread t scans bin 255 - t, so its inclusive prefix is
  // S(255 - t) = candidates in bins >= 255 - t
  const int incl = wave_incl_scan((int)binv[255 - t]);
  if (lane == kWave - 1) wave_sum_s[wave] = (unsigned)incl;
  __syncthreads();
  unsigned before = 0u;
  for (int v = 0; v < wave; ++v) before += wave_sum_s[v];
  sfx[255 - t] = before + (unsigned)incl;
  if (t == 0) sfx[256] = 0u;
  __syncthreads();
  // the digit is the highest bin bb (bb >= 1) with S(bb) >= need, else 0;
  // above = S(bb + 1).  S is non-increasing, so exactly one thread matches.
  const unsigned prefix = pass ? state[2 * kv] : 0u;
  const unsigned need = pass ? state[2 * kv + 1] : (unsigned)m;
  const int bb = t;
  const bool here = bb >= 1 ? (sfx[bb] >= need && sfx[bb + 1] < need) : (sfx[1] < need);
  if (here) {
    state[2 * kv] = prefix | ((unsigned)bb << (24 - 8 * pass));
    state[2 * kv + 1] = need - sfx[bb + 1];
  }
}

// COUNT: write (kept-above-T plus forced, equal-to-T candidates) of the chunk.
// !COUNT: emit the chunk's part of the ascending list.
template <bool COUNT>
__global__ __launch_bounds__(kTopkThreads) void sel_topk_chunk_kernel(
    const float* __restrict__ scores, int n, int w, int n_sink, int k_keep_all, int ragged,
    HeadInts k_heads, int stride, const unsigned* __restrict__ state, int* __restrict__ counts,
    int32_t* __restrict__ idx) {
  __shared__ int wave_tot[kTopkWaves];
  __shared__ int sh_pos, sh_ties;
  const int ch = blockIdx.x, kv = blockIdx.y, C = gridDim.x;
  const float* S = scores + (size_t)kv * n;
  const int k_keep = topk_budget(ragged, k_heads, k_keep_all, kv);
  int32_t* out = idx + (size_t)kv * stride;
  const int q0 = ch * kTopkChunk, q1 = min(n, q0 + kTopkChunk);
  if (k_keep >= n) {  // identity selection
    if (!COUNT)
      for (int j = q0 + threadIdx.x; j < q1; j += kTopkThreads) out[j] = j;
    return;
  }
  const int m = k_keep - n_sink - w;
  const int c0 = n_sink, c1 = n - w;
  const unsigned T = m > 0 ? state[2 * kv] : 0u;
  const int need = m > 0 ? (int)state[2 * kv + 1] : 0;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  // one 64-position block per wave and step (the chunk is 4096 positions: 4 blocks per wave)
  constexpr int EU = kTopkChunk / kTopkThreads;
  const int p0 = q0 + wave * kWave * EU;
  auto key_at = [&](int j) { return order_key(S[min(j, n - 1)]); };
  unsigned kk[EU];
#pragma unroll
  for (int u = 0; u < EU; ++u) kk[u] = key_at(p0 + kWave * u + lane);
  int n_take = 0, n_eq = 0;  // wave totals (uniform)
#pragma unroll
  for (int u = 0; u < EU; ++u) {
    const int j = p0 + kWave * u + lane;
    const bool valid = j < q1;
    const bool forced = valid && (j < c0 || j >= c1);
    const bool cand = valid && !forced && m > 0;
    n_take += __popcll(__ballot(forced || (cand && kk[u] > T)));
    n_eq += __popcll(__ballot(cand && kk[u] == T));
  }
  if (COUNT) {
    int take_total, eq_total;
    (void)block_excl_sum(lane == 0 ? n_take : 0, wave_tot, take_total);
    (void)block_excl_sum(lane == 0 ? n_eq : 0, wave_tot, eq_total);
    if (threadIdx.x == 0) {
      counts[2 * ((size_t)kv * C + ch)] = take_total;
      counts[2 * ((size_t)kv * C + ch) + 1] = eq_total;
    }
    return;
  }
  // this chunk's list offset and ties from the chunks before it
  if (threadIdx.x == 0) {
    int pos = 0, eq_before = 0;
    for (int c = 0; c < ch; ++c) {
      const int take_c = counts[2 * ((size_t)kv * C + c)], eq_c = counts[2 * ((size_t)kv * C + c) + 1];
      pos += take_c + max(0, min(eq_c, need - eq_before));
      eq_before += eq_c;
    }
    sh_pos = pos;
    sh_ties = max(0, need - eq_before);  // ties still to keep, this chunk first
  }
  __syncthreads();
  const int chunk_ties = sh_ties;
  int eq_total;
  const int eq_before = block_excl_sum(lane == 0 ? n_eq : 0, wave_tot, eq_total);
  const int eq_wave = __shfl(eq_before, 0);
  const int ties = max(0, min(n_eq, chunk_ties - eq_wave));  // ties this wave keeps
  int take_total;
  const int pos_before = block_excl_sum(lane == 0 ? n_take + ties : 0, wave_tot, take_total);
  int pos = sh_pos + __shfl(pos_before, 0), eq_seen = 0;
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int u = 0; u < EU; ++u) {
    const int j = p0 + kWave * u + lane;
    const bool valid = j < q1;
    const bool forced = valid && (j < c0 || j >= c1);
    const bool cand = valid && !forced && m > 0;
    const bool eq = cand && kk[u] == T;
    const unsigned long long eqm = __ballot(eq);
    const bool take = forced || (cand && kk[u] > T) ||
                      (eq && eq_seen + __popcll(eqm & below) < ties);
    const unsigned long long tm = __ballot(take);
    if (take) {
      const int p = pos + __popcll(tm & below);
      if (p < k_keep) out[p] = j;  // p < k_keep always; guard anyway
    }
    pos += __popcll(tm);
    eq_seen += __popcll(eqm);
  }
}

template <typename KT, int DH>
static void select_typed(const SelectArgs& a, hipStream_t s) {
  const int G = a.h_q / a.h_kv;
  const float scale_log2 = (1.0f / sqrtf((float)DH)) * 1.44269504088896340736f;
  const KT* k = (const KT*)a.k;
  if (!a.skip_scoring) {
    dim3 grid(a.n_chunks, a.h_kv);
    constexpr bool kMfma = sizeof(KT) == 2;  // bf16 caches: matrix cores
    const dim3 mgrid((a.n_chunks + kSelSub - 1) / kSelSub, a.h_kv);
    if constexpr (kMfma)
      launch_kernel(K_SEL_LSE, sel_lse_partial_mfma_kernel<DH>, mgrid, dim3(kSelThreads), 0, s,
                    (const bf16_t*)k, a.cap_full, a.n, a.q_win, a.w, G, scale_log2, a.n_chunks,
                    a.lse_part);
    else
      launch_kernel(K_SEL_LSE, sel_lse_partial_kernel<KT, DH>, grid, dim3(kSelThreads), 0, s, k,
                    a.cap_full, a.n, a.q_win, a.w, G, scale_log2, a.n_chunks, a.lse_part);
    const int nq = a.h_kv * G * a.w;  // one wave each, four per workgroup
    launch_kernel(K_SEL_LSE_FINAL, sel_lse_final_kernel, dim3((nq + 3) / 4), dim3(256), 0, s,
                  (const float*)a.lse_part, a.n_chunks, G, a.w, a.h_kv, a.lse);
    if constexpr (kMfma)
      launch_kernel(K_SEL_SCORE, sel_score_mfma_kernel<DH>, mgrid, dim3(kSelThreads), 0, s,
                    (const bf16_t*)k, a.cap_full, a.n, a.q_win, a.w, G, scale_log2,
                    (const float*)a.lse, a.scores);
    else
      launch_kernel(K_SEL_SCORE, sel_score_kernel<KT, DH>, grid, dim3(kSelThreads), 0, s, k,
                    a.cap_full, a.n, a.q_win, a.w, G, scale_log2, (const float*)a.lse, a.scores);
  }
  // per-head kept counts (one count for all heads unless the budgets are ragged)
  HeadInts k_eff_heads{};
  int k_eff = a.k_keep < a.n ? a.k_keep : a.n, k_max = k_eff;
  if (a.ragged) {
    k_max = 0;
    for (int h = 0; h < a.h_kv; ++h) {
      k_eff_heads.v[h] = a.k_heads.v[h] < a.n ? a.k_heads.v[h] : a.n;
      if (k_eff_heads.v[h] > k_max) k_max = k_eff_heads.v[h];
    }
  }
  const int stride = a.ragged ? a.idx_stride : k_eff;
  const int C = (a.n + kTopkChunk - 1) / kTopkChunk;
  if (C <= 2 || C > kTopkMaxChunks || !a.topk_ws) {
    launch_kernel(K_SEL_TOPK, sel_topk_kernel, dim3(a.h_kv), dim3(kTopkThreads), 0, s,
                  (const float*)a.scores, a.n, a.w, a.n_sink, a.k_keep, a.ragged, a.k_heads,
                  stride, a.idx);
  } else {
    // workspace: hist [h_kv, C, 256], counts [h_kv, C, 2], state [h_kv, 2]
    unsigned* hist = a.topk_ws;
    int* counts = reinterpret_cast<int*>(hist + (size_t)a.h_kv * kTopkMaxChunks * 256);
    unsigned* state = reinterpret_cast<unsigned*>(counts + (size_t)a.h_kv * kTopkMaxChunks * 2);
    for (int pass = 0; pass < 4; ++pass) {
      launch_kernel(K_SEL_TOPK, sel_topk_hist_kernel, dim3(C, a.h_kv), dim3(kTopkThreads), 0, s,
                    (const float*)a.scores, a.n, a.w, a.n_sink, a.k_keep, a.ragged, a.k_heads,
                    pass, (const unsigned*)state, hist);
      launch_kernel(K_SEL_TOPK, sel_topk_pick_kernel, dim3(a.h_kv), dim3(256), 0, s, a.n, a.w,
                    a.n_sink, a.k_keep, a.ragged, a.k_heads, pass, C, state,
                    (const unsigned*)hist);
    }
    launch_kernel(K_SEL_TOPK, sel_topk_chunk_kernel<true>, dim3(C, a.h_kv), dim3(kTopkThreads), 0,
                  s, (const float*)a.scores, a.n, a.w, a.n_sink, a.k_keep, a.ragged, a.k_heads,
                  stride, (const unsigned*)state, counts, a.idx);
    launch_kernel(K_SEL_TOPK, sel_topk_chunk_kernel<false>, dim3(C, a.h_kv), dim3(kTopkThreads),
                  0, s, (const float*)a.scores, a.n, a.w, a.n_sink, a.k_keep, a.ragged, a.k_heads,
                  stride, (const unsigned*)state, counts, a.idx);
  }
  constexpr int P = DH * (int)sizeof(KT) / 16;
  dim3 ggrid((k_max * P + 255) / 256, a.h_kv);
  launch_kernel(K_SEL_GATHER, sel_gather_kernel<KT, DH>, ggrid, dim3(256), 0, s, k,
                (const KT*)a.v, a.cap_full, (const int32_t*)a.idx, k_eff, a.ragged, k_eff_heads,
                stride, (KT*)a.k_sel, (KT*)a.v_sel, a.cap_sel);
}

void launch_select(const SelectArgs& a, int kv_dtype, hipStream_t s) {
  if (a.dh == 64) {
    if (kv_dtype == 1) select_typed<bf16_t, 64>(a, s);
    else select_typed<float, 64>(a, s);
  } else {
    if (kv_dtype == 1) select_typed<bf16_t, 128>(a, s);
    else select_typed<float, 128>(a, s);
  }
}

// ------------------------------------------------------------------ k-th smallest
// Order statistic of non-negative float32 values (their bit patterns order
// like the values): four 8-bit digit passes, each a grid-wide histogram of the
// values that match the digits found so far, then one thread picks the digit.
// state[0] = prefix found so far, state[1] = rank still needed within it.
__global__ void kth_init_kernel(unsigned* hist, unsigned* state, unsigned k) {
  for (int b = threadIdx.x; b < 256; b += blockDim.x) hist[b] = 0u;
  if (threadIdx.x == 0) {
    state[0] = 0u;
    state[1] = k;
  }
}

__global__ __launch_bounds__(256) void kth_hist_kernel(const float* __restrict__ vals, size_t n,
                                                       int pass, const unsigned* __restrict__ state,
                                                       unsigned* __restrict__ hist) {
  __shared__ unsigned h[256];
  h[threadIdx.x] = 0u;
  __syncthreads();
  const unsigned prefix = state[0];
  const int shift = 24 - 8 * pass;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    const float f = vals[i];
    const unsigned key = f == 0.f ? 0u : __float_as_uint(f);
    if (pass == 0 || (key >> (shift + 8)) == (prefix >> (shift + 8)))
      atomicAdd(&h[(key >> shift) & 255u], 1u);
  }
  __syncthreads();
  if (h[threadIdx.x]) atomicAdd(&hist[threadIdx.x], h[threadIdx.x]);
}

__global__ void kth_pick_kernel(int pass, unsigned* hist, unsigned* state, float* out) {
  if (threadIdx.x != 0) return;
  const int shift = 24 - 8 * pass;
  unsigned need = state[1], below = 0;
  int b = 0;
  for (; b < 255; ++b) {
    if (below + hist[b] >= need) break;
    below += hist[b];
  }
  state[0] |= (unsigned)b << shift;
  state[1] = need - below;
  for (int i = 0; i < 256; ++i) hist[i] = 0u;
  if (pass == 3) *out = __uint_as_float(state[0]);
}

__global__ void fill_kernel(float* out, float v) { *out = v; }

void launch_kth_smallest(const float* vals, size_t n, size_t k, unsigned* hist, unsigned* state,
                         float* out, hipStream_t s) {
  if (k == 0) {
    launch_kernel(-1, fill_kernel, dim3(1), dim3(1), 0, s, out, -1.0f);
    return;
  }
  launch_kernel(-1, kth_init_kernel, dim3(1), dim3(256), 0, s, hist, state, (unsigned)k);
  size_t blocks = (n + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  for (int pass = 0; pass < 4; ++pass) {
    launch_kernel(K_KTH, kth_hist_kernel, dim3((unsigned)blocks), dim3(256), 0, s, vals, n, pass,
                  (const unsigned*)state, hist);
    launch_kernel(-1, kth_pick_kernel, dim3(1), dim3(64), 0, s, pass, hist, state, out);
  }
}

}  // namespace sd
