// Split-K GQA decode attention (gfx950, wave64).
//
// "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding"
// reads every cache -- full in dense mode, gathered in KV mode -- through one
// split-K decoding kernel (§1, §4.1), and §4.4 shows why the dense baseline
// must be that efficient path.  This is this library's own design for CDNA:
//
//   one launch, grid (splits, KV heads): a workgroup owns a contiguous chunk
//   of rows of one KV head and serves all G query heads of the group, so each
//   K/V byte is read once.  A row of d_h elements is spread over d_h/8 lanes
//   (16-byte loads); the wave holds 64/(d_h/8) row slots, and each slot keeps
//   U rows in flight per iteration (U = 4 with four query heads per KV head:
//   occupancy 3), so a workgroup streams U*16 consecutive rows of K and of V
//   per iteration (the chunk is read in address order).
//   Every lane group keeps its own online-softmax state (max, sum, acc) in the
//   log2 domain; at the end the groups and the four waves merge their states
//   and write one (m, l, acc[d_h]) per query head and split.
//
//   A second, small launch merges the splits, one workgroup per query head:
//   out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s, lse = (M + log2 L) ln 2,
//   splits in order, so the result does not depend on scheduling.  The launch
//   boundary makes the partials visible to every XCD; measured on MI355X it is
//   cheaper than a hand-off inside one launch (coherent stores, a wait for
//   their acknowledgement, a ticket and coherent loads are three memory round
//   trips).
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace sd {

constexpr int kAttnThreads = 256;
constexpr int kMaxSplits = 128;  // splits per KV head (the merge holds one column of them in VGPRs)
constexpr int kAttnWaves = kAttnThreads / kWave;

template <typename KT, int DH, int G, int U>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(
    const float* __restrict__ q, const KT* __restrict__ K, const KT* __restrict__ V, int cap,
    int n_ctx, int sink, int shift, int kv_div, int ragged, HeadInts lens, float scale_log2,
    int chunk, int n_splits, float* __restrict__ pm, float* __restrict__ pl,
    float* __restrict__ pacc) {
  constexpr int LPR = DH / 8;          // lanes per row
  constexpr int RPW = kWave / LPR;     // row slots per wave
  constexpr int SLOTS = kAttnWaves * RPW;
  __shared__ float sm_m[kAttnWaves][G], sm_l[kAttnWaves][G];
  __shared__ float sm_acc[kAttnWaves][G][DH];

  const int split = blockIdx.x, kv = blockIdx.y;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int sub = lane % LPR;
  const int slot = wave * RPW + lane / LPR;
  // rows of this KV head: n_ctx, or its own count under ragged budgets (a
  // split past the end has no rows and writes the empty partial)
  const int rows = ragged ? lens.v[(kv / kv_div) & (kMaxKvHeads - 1)] : n_ctx;
  const int r0 = split * chunk;
  const int r1 = min(rows, r0 + chunk);
  // logical row j is physical row j, or j + shift from `sink` on (a window of
  // sinks plus recent rows read in place); query-head group kv reads KV head
  // kv / kv_div (kv_div > 1: one workgroup per query head)
  const KT* Kb = K + (size_t)(kv / kv_div) * cap * DH + 8 * sub;
  const KT* Vb = V + (size_t)(kv / kv_div) * cap * DH + 8 * sub;
  auto phys = [&](int jj) { return (size_t)(jj + (jj >= sink ? shift : 0)); };

  // first rows in flight before the query is read
  Vec8<KT> kr[U], vr[U];
  int j = r0 + slot;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int jj = j + u * SLOTS;
    if (jj < r1) {
      kr[u].load(Kb + phys(jj) * DH);
      vr[u].load(Vb + phys(jj) * DH);
    }
  }

  float qv[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    load8f(q + (size_t)(kv * G + g) * DH + 8 * sub, qv[g]);
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[g][e] *= scale_log2;
  }
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }

  for (; j < r1; j += U * SLOTS) {
    float p[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = j + u * SLOTS < r1;
      float kf[8];
      kr[u].to_float(kf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) t = fmaf(kf[e], qv[g][e], t);
        t = group_sum<LPR>(t);
        p[u][g] = ok ? t : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mb = p[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u) mb = fmaxf(mb, p[u][g]);
      const float mn = fmaxf(m[g], mb);  // finite: row j itself is valid
      const float alpha = exp2f(m[g] - mn);
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u][g] = exp2f(p[u][g] - mn);
        ps += p[u][g];
      }
      l[g] = fmaf(l[g], alpha, ps);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
      m[g] = mn;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[8];
      vr[u].to_float(vf);
      if (!(j + u * SLOTS < r1))
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[e] = 0.f;  // never loaded: keep NaN/Inf out
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(p[u][g], vf[e], acc[g][e]);
    }
    // next rows
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j + U * SLOTS + u * SLOTS;
      if (jj < r1) {
        kr[u].load(Kb + phys(jj) * DH);
        vr[u].load(Vb + phys(jj) * DH);
      }
    }
  }

  // merge the row slots of the wave (lane groups that differ in lane / LPR)
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      const float mn = fmaxf(m[g], mo);
      const float a1 = m[g] == -INFINITY ? 0.f : exp2f(m[g] - mn);
      const float a2 = mo == -INFINITY ? 0.f : exp2f(mo - mn);
      l[g] = l[g] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ao = __shfl_xor(acc[g][e], off);
        acc[g][e] = acc[g][e] * a1 + ao * a2;
      }
      m[g] = mn;
    }
  }
  if (lane < LPR) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (lane == 0) {
        sm_m[wave][g] = m[g];
        sm_l[wave][g] = l[g];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_acc[wave][g][8 * lane + e] = acc[g][e];
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < G * DH; t += kAttnThreads) {
    const int g = t / DH, c = t - g * DH;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, sm_m[w][g]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float a = sm_m[w][g] == -INFINITY ? 0.f : exp2f(sm_m[w][g] - M);
      L = fmaf(sm_l[w][g], a, L);
      A = fmaf(sm_acc[w][g][c], a, A);
    }
    const size_t hs = (size_t)(kv * G + g) * n_splits + split;
    pacc[hs * DH + c] = A;
    if (c == 0) {
      pm[hs] = M;
      pl[hs] = L;
    }
  }
}

// One workgroup per query head, one thread per column: every split's value of
// the thread's column is loaded before the first is used (one memory round
// trip); wave 0 turns the split maxima into weights.
template <int DH, int CAP>
__global__ __launch_bounds__(DH) void attn_merge_kernel(const float* __restrict__ pm,
                                                        const float* __restrict__ pl,
                                                        const float* __restrict__ pacc,
                                                        int n_splits, float* __restrict__ out,
                                                        float* __restrict__ lse) {
  __shared__ float w_s[CAP];
  __shared__ float inv_l, big_m, big_l;
  const int h = blockIdx.x, c = threadIdx.x;
  const float* base = pacc + (size_t)h * n_splits * DH + c;
  float v[CAP];
#pragma unroll
  for (int sp = 0; sp < CAP; ++sp)
    v[sp] = sp < n_splits ? base[(size_t)sp * DH] : 0.f;
  if (threadIdx.x < kWave) {  // wave 0: split weights, CAP / 64 splits per lane
    constexpr int PL = CAP / kWave;
    const int lane = threadIdx.x;
    float mi[PL], li[PL];
#pragma unroll
    for (int k = 0; k < PL; ++k) {
      const int sp = lane + k * kWave;
      mi[k] = sp < n_splits ? pm[(size_t)h * n_splits + sp] : -INFINITY;
      li[k] = sp < n_splits ? pl[(size_t)h * n_splits + sp] : 0.f;
    }
    float mm = mi[0];
#pragma unroll
    for (int k = 1; k < PL; ++k) mm = fmaxf(mm, mi[k]);
    const float M = wave_max(mm);
    float wl = 0.f;
#pragma unroll
    for (int k = 0; k < PL; ++k) {
      const float wi = mi[k] == -INFINITY ? 0.f : exp2f(mi[k] - M);
      w_s[lane + k * kWave] = wi;
      wl = fmaf(wi, li[k], wl);
    }
    const float L = wave_sum(wl);
    if (lane == 0) {
      big_m = M;
      big_l = L;
      inv_l = 1.0f / L;
    }
  }
  __syncthreads();
  float A = 0.f;
#pragma unroll
  for (int sp = 0; sp < CAP; ++sp)
    if (sp < n_splits) A = fmaf(w_s[sp], v[sp], A);
  out[(size_t)h * DH + c] = A * inv_l;
  if (lse && c == 0) lse[h] = (big_m + log2f(big_l)) * 0.69314718055994530942f;
}

template <typename KT, int DH>
static void attn_dh(const AttnArgs& a, hipStream_t s) {
  // per_query_head: one workgroup (group of one) per query head, reading KV head h / G
  const int G = a.per_query_head ? 1 : a.h_q / a.h_kv;
  const int kv_div = a.per_query_head ? a.h_q / a.h_kv : 1;
  const int groups = a.per_query_head ? a.h_q : a.h_kv;
  const float scale_log2 = a.scale * 1.44269504088896340736f;
  dim3 grid(a.n_splits, groups);
  const KT* k = (const KT*)a.k;
  const KT* v = (const KT*)a.v;
#define SD_ATTN_G(GG, UU)                                                                   \
  launch_kernel(K_ATTN_PARTIAL, attn_kernel<KT, DH, GG, UU>, grid, dim3(kAttnThreads), 0, s, \
                a.q, k, v, a.cap, a.n_ctx, a.sink, a.shift, kv_div, a.ragged, a.lens, scale_log2,      \
                a.chunk, a.n_splits, a.pm, a.pl, a.pacc)
  switch (G) {
    case 1: SD_ATTN_G(1, 8); break;
    case 2: SD_ATTN_G(2, 8); break;
    case 4: SD_ATTN_G(4, 4); break;
    default: SD_ATTN_G(8, 4); break;
  }
#undef SD_ATTN_G
  if (a.n_splits <= 64)
    launch_kernel(K_ATTN_COMBINE, attn_merge_kernel<DH, 64>, dim3(a.h_q), dim3(DH), 0, s, a.pm,
                  a.pl, a.pacc, a.n_splits, a.out, a.lse);
  else
    launch_kernel(K_ATTN_COMBINE, attn_merge_kernel<DH, kMaxSplits>, dim3(a.h_q), dim3(DH), 0, s,
                  a.pm, a.pl, a.pacc, a.n_splits, a.out, a.lse);
}

void launch_attn(const AttnArgs& a, int kv_dtype, hipStream_t s) {
  if (a.dh == 64) {
    if (kv_dtype == 1) attn_dh<bf16_t, 64>(a, s);
    else attn_dh<float, 64>(a, s);
  } else {
    if (kv_dtype == 1) attn_dh<bf16_t, 128>(a, s);
    else attn_dh<float, 128>(a, s);
  }
}

}  // namespace sd
