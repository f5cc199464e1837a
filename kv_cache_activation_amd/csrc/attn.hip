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
//   U rows in flight per iteration, so a workgroup streams U*16 consecutive
//   rows of K and of V per iteration (the chunk is read in address order).
//   Every lane group keeps its own online-softmax state (max, sum, acc) in the
//   log2 domain; at the end the groups and the four waves merge their states
//   and write one (m, l, acc[d_h]) per query head and split.
//
//   The last workgroup to finish for a KV head (device-scope ticket counter,
//   zeroed before the launch) merges that head's splits:
//   out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s, lse = (M + log2 L) ln 2,
//   splits in order, so the result does not depend on scheduling.  Partials
//   travel between workgroups through device-scope coherent stores and loads,
//   not through a cache-flushing fence.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace sd {

constexpr int kAttnThreads = 256;
constexpr int kMaxSplits = 64;  // splits per KV head (the merge holds their weights in one wave)
constexpr int kAttnWaves = kAttnThreads / kWave;

// Merge of the split partials of KV head kv by one workgroup: every load is
// issued before the first one is consumed (one memory round trip), then
// out = sum_s w_s acc_s / sum_s w_s l_s with w_s = 2^(m_s - M), in split order.
template <int G, int DH>
__device__ __forceinline__ void merge_splits(const float* __restrict__ pm,
                                             const float* __restrict__ pl,
                                             const float* __restrict__ pacc, int kv, int n_splits,
                                             float* __restrict__ out, float* __restrict__ lse,
                                             float (*w_s)[kMaxSplits], float* inv_l, float* big_m,
                                             float* big_l) {
  constexpr int OUTS = G * DH;        // (head, column) outputs of this KV head
  constexpr int PER = 2;              // outputs per thread and pass
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  // split maxima and sums: wave w handles heads w, w + 4, ...
  float mi[(G + kAttnWaves - 1) / kAttnWaves], li[(G + kAttnWaves - 1) / kAttnWaves];
#pragma unroll
  for (int k = 0; k < (G + kAttnWaves - 1) / kAttnWaves; ++k) {
    const int g = wave + k * kAttnWaves;
    const size_t h0 = (size_t)(kv * G + g) * n_splits;
    const bool ok = g < G && lane < n_splits;
    mi[k] = ok ? coherent_load(pm + h0 + lane) : -INFINITY;
    li[k] = ok ? coherent_load(pl + h0 + lane) : 0.f;
  }
  float v[PER][kMaxSplits];
  auto load_pass = [&](int o0) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int o = o0 + k * kAttnThreads;
      const int g = o / DH, c = o - (o / DH) * DH;
      const float* base = pacc + (size_t)(kv * G + g) * n_splits * DH + c;
#pragma unroll
      for (int sp = 0; sp < kMaxSplits; ++sp)
        v[k][sp] = (o < OUTS && sp < n_splits) ? coherent_load(base + (size_t)sp * DH) : 0.f;
    }
  };
  auto finish_pass = [&](int o0) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int o = o0 + k * kAttnThreads;
      if (o < OUTS) {
        const int g = o / DH, c = o - (o / DH) * DH;
        float A = 0.f;
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp)
          if (sp < n_splits) A = fmaf(w_s[g][sp], v[k][sp], A);
        out[(size_t)(kv * G + g) * DH + c] = A * inv_l[g];
        if (lse && c == 0) lse[kv * G + g] = (big_m[g] + log2f(big_l[g])) * 0.69314718055994530942f;
      }
    }
  };
  load_pass(threadIdx.x);  // first pass in flight while the weights are formed
#pragma unroll
  for (int k = 0; k < (G + kAttnWaves - 1) / kAttnWaves; ++k) {
    const int g = wave + k * kAttnWaves;
    if (g < G) {  // wave-uniform
      const float M = wave_max(mi[k]);
      const float wi = mi[k] == -INFINITY ? 0.f : exp2f(mi[k] - M);
      const float L = wave_sum(wi * li[k]);
      if (lane < n_splits) w_s[g][lane] = wi;
      if (lane == 0) {
        big_m[g] = M;
        big_l[g] = L;
        inv_l[g] = 1.0f / L;
      }
    }
  }
  __syncthreads();  // every thread of the workgroup reaches this
  finish_pass(threadIdx.x);
  for (int o0 = threadIdx.x + PER * kAttnThreads; o0 < OUTS; o0 += PER * kAttnThreads) {
    load_pass(o0);
    finish_pass(o0);
  }
}

template <typename KT, int DH, int G, int U>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(
    const float* __restrict__ q, const KT* __restrict__ K, const KT* __restrict__ V, int cap,
    int n_ctx, float scale_log2, int chunk, int n_splits, float* __restrict__ pm,
    float* __restrict__ pl, float* __restrict__ pacc, unsigned* __restrict__ counters,
    float* __restrict__ out, float* __restrict__ lse) {
  constexpr int LPR = DH / 8;          // lanes per row
  constexpr int RPW = kWave / LPR;     // row slots per wave
  constexpr int SLOTS = kAttnWaves * RPW;
  __shared__ float sm_m[kAttnWaves][G], sm_l[kAttnWaves][G];
  __shared__ float sm_acc[kAttnWaves][G][DH];

  const int split = blockIdx.x, kv = blockIdx.y;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int sub = lane % LPR;
  const int slot = wave * RPW + lane / LPR;
  const int r0 = split * chunk;
  const int r1 = min(n_ctx, r0 + chunk);
  const KT* Kb = K + (size_t)kv * cap * DH + 8 * sub;
  const KT* Vb = V + (size_t)kv * cap * DH + 8 * sub;

  // first rows in flight before the query is read
  Vec8<KT> kr[U], vr[U];
  int j = r0 + slot;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int jj = j + u * SLOTS;
    if (jj < r1) {
      kr[u].load(Kb + (size_t)jj * DH);
      vr[u].load(Vb + (size_t)jj * DH);
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
        kr[u].load(Kb + (size_t)jj * DH);
        vr[u].load(Vb + (size_t)jj * DH);
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
    coherent_store(pacc + hs * DH + c, A);
    if (c == 0) {
      coherent_store(pm + hs, M);
      coherent_store(pl + hs, L);
    }
  }

  // ---- last workgroup of this KV head merges all splits
  __shared__ int last_s;
  __shared__ float w_s[G][kMaxSplits];
  __shared__ float inv_l[G], big_m[G], big_l[G];
  stores_done();
  __syncthreads();
  if (threadIdx.x == 0) last_s = last_arrival(&counters[kv], (unsigned)n_splits);
  __syncthreads();
  if (!last_s) return;
  merge_splits<G, DH>(pm, pl, pacc, kv, n_splits, out, lse, w_s, inv_l, big_m, big_l);
}

__global__ void zero_u32_kernel(unsigned* __restrict__ p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

template <typename KT, int DH>
static void attn_dh(const AttnArgs& a, hipStream_t s) {
  const int G = a.h_q / a.h_kv;
  const float scale_log2 = a.scale * 1.44269504088896340736f;
  dim3 grid(a.n_splits, a.h_kv);
  const KT* k = (const KT*)a.k;
  const KT* v = (const KT*)a.v;
  if (a.zero_counters) zero_u32_kernel<<<1, 64, 0, s>>>(a.counters, a.h_kv);
#define SD_ATTN_G(GG, UU)                                                                   \
  attn_kernel<KT, DH, GG, UU><<<grid, kAttnThreads, 0, s>>>(                               \
      a.q, k, v, a.cap, a.n_ctx, scale_log2, a.chunk, a.n_splits, a.pm, a.pl, a.pacc,      \
      a.counters, a.out, a.lse)
  ProfScope prof(K_ATTN_PARTIAL, s);
  switch (G) {
    case 1: SD_ATTN_G(1, 8); break;
    case 2: SD_ATTN_G(2, 8); break;
    case 4: SD_ATTN_G(4, 8); break;
    default: SD_ATTN_G(8, 4); break;
  }
#undef SD_ATTN_G
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
