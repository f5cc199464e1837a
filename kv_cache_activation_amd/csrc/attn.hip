// Split-K GQA decode attention (gfx950, wave64).
//
// "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding"
// reads every cache -- full in dense mode, gathered in KV mode -- through one
// split-K decoding kernel (§1, §4.1), and §4.4 shows why the dense baseline
// must be that efficient path.  This is this library's own design for CDNA:
//
//   partial kernel, grid (splits, KV heads): a workgroup owns a contiguous
//   chunk of rows of one KV head and serves all G query heads of the group, so
//   each K/V byte is read once.  A row of d_h elements is spread over d_h/8
//   lanes (16-byte loads); the wave holds 64/(d_h/8) rows at once, each lane
//   group keeping its own online-softmax state (max, sum, acc) in the log2
//   domain.  Two rows per lane group are in flight per iteration.  At the end
//   the lane groups and the four waves merge their states and write one
//   (m, l, acc[d_h]) per query head and split.
//
//   The last workgroup to finish for a KV head (device-scope ticket counter,
//   zeroed before the launch) merges that head's split partials:
//   out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s, lse = (M + log2 L) ln 2,
//   splits in order, so the result does not depend on scheduling.  All split
//   loads of that merge are issued together (at most kMaxSplits per head).
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace sd {

constexpr int kAttnThreads = 256;
constexpr int kMaxSplits = 64;  // splits per KV head (the merge holds them in VGPRs)
constexpr int kAttnWaves = kAttnThreads / kWave;

template <typename KT, int DH, int G>
__global__ __launch_bounds__(kAttnThreads) void attn_partial_kernel(
    const float* __restrict__ q, const KT* __restrict__ K, const KT* __restrict__ V, int cap,
    int n_ctx, float scale_log2, int chunk, int n_splits, float* __restrict__ pm,
    float* __restrict__ pl, float* __restrict__ pacc, unsigned* __restrict__ counters,
    float* __restrict__ out, float* __restrict__ lse) {
  constexpr int LPR = DH / 8;          // lanes per row
  constexpr int RPW = kWave / LPR;     // row slots per wave
  constexpr int SLOTS = kAttnWaves * RPW;
  constexpr int U = 4;                 // rows in flight per slot
  __shared__ float sm_m[kAttnWaves][G], sm_l[kAttnWaves][G];
  __shared__ float sm_acc[kAttnWaves][G][DH];

  const int split = blockIdx.x, kv = blockIdx.y;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int sub = lane % LPR;
  const int slot = wave * RPW + lane / LPR;
  const int r0 = split * chunk;
  const int r1 = min(n_ctx, r0 + chunk);

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
  const KT* Kb = K + (size_t)kv * cap * DH + 8 * sub;
  const KT* Vb = V + (size_t)kv * cap * DH + 8 * sub;

  for (int j = r0 + slot; j < r1; j += U * SLOTS) {
    Vec8<KT> kr[U], vr[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j + u * SLOTS;
      ok[u] = jj < r1;
      if (ok[u]) {
        kr[u].load(Kb + (size_t)jj * DH);
        vr[u].load(Vb + (size_t)jj * DH);
      }
    }
    float sc[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[8];
      kr[u].to_float(kf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) t = fmaf(kf[e], qv[g][e], t);
        t = group_sum<LPR>(t);
        sc[u][g] = ok[u] ? t : -INFINITY;
      }
    }
    float vf[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      vr[u].to_float(vf[u]);
      if (!ok[u])
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[u][e] = 0.f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mb = sc[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u) mb = fmaxf(mb, sc[u][g]);
      const float mn = fmaxf(m[g], mb);  // finite: row j itself is valid
      const float alpha = exp2f(m[g] - mn);
      float p[U];
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u] = exp2f(sc[u][g] - mn);
        ps += p[u];
      }
      l[g] = fmaf(l[g], alpha, ps);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float a = acc[g][e] * alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) a = fmaf(p[u], vf[u][e], a);
        acc[g][e] = a;
      }
      m[g] = mn;
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

  // ---- last workgroup of this KV head merges all splits
  __shared__ int last_s;
  __shared__ float w_s[G][kMaxSplits], l_s[G][kMaxSplits];
  __shared__ float big_m[G], big_l[G];
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) last_s = atomicAdd(&counters[kv], 1u) == (unsigned)(n_splits - 1);
  __syncthreads();
  if (!last_s) return;
  __threadfence();
  for (int t = threadIdx.x; t < G * n_splits; t += kAttnThreads) {
    const int g = t / n_splits, sp = t - g * n_splits;
    const size_t hs = (size_t)(kv * G + g) * n_splits + sp;
    w_s[g][sp] = __builtin_nontemporal_load(pm + hs);
    l_s[g][sp] = __builtin_nontemporal_load(pl + hs);
  }
  __syncthreads();
  for (int g = wave; g < G; g += kAttnWaves) {
    const float mi = lane < n_splits ? w_s[g][lane] : -INFINITY;
    const float M = wave_max(mi);
    const float wi = mi == -INFINITY ? 0.f : exp2f(mi - M);
    const float L = wave_sum(lane < n_splits ? wi * l_s[g][lane] : 0.f);
    if (lane < n_splits) w_s[g][lane] = wi;
    if (lane == 0) {
      big_m[g] = M;
      big_l[g] = L;
    }
  }
  __syncthreads();
  // thread (split group sg, column quad cq) accumulates its splits' float4s of
  // every head; then the split groups are summed through LDS in group order
  constexpr int NQ = DH / 4;                 // float4 column quads per row
  constexpr int GROUPS = kAttnThreads / NQ;  // split groups
  constexpr int ITERS = kMaxSplits / GROUPS;
  const int cq = threadIdx.x % NQ, sg = threadIdx.x / NQ;
  __shared__ float red[GROUPS * G * DH];
  for (int g = 0; g < G; ++g) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    f32x4 v[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int sp = sg + it * GROUPS;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      v[it] = sp < n_splits ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(
                                  pacc + ((size_t)(kv * G + g) * n_splits + sp) * DH) + cq)
                            : z;
    }
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int sp = sg + it * GROUPS;
      if (sp < n_splits) a += w_s[g][sp] * v[it];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) red[sg * G * DH + g * DH + 4 * cq + e] = a[e];
  }
  __syncthreads();
  for (int o = threadIdx.x; o < G * DH; o += kAttnThreads) {
    const int g = o / DH, c = o - g * DH;
    float A = 0.f;
#pragma unroll
    for (int grp = 0; grp < GROUPS; ++grp) A += red[grp * G * DH + o];
    out[(size_t)(kv * G + g) * DH + c] = A / big_l[g];
    if (lse && c == 0) lse[kv * G + g] = (big_m[g] + log2f(big_l[g])) * 0.69314718055994530942f;
  }
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
#define SD_ATTN_G(GG)                                                                      \
  attn_partial_kernel<KT, DH, GG><<<grid, kAttnThreads, 0, s>>>(                           \
      a.q, k, v, a.cap, a.n_ctx, scale_log2, a.chunk, a.n_splits, a.pm, a.pl, a.pacc,      \
      a.counters, a.out, a.lse)
  ProfScope prof(K_ATTN_PARTIAL, s);
  switch (G) {
    case 1: SD_ATTN_G(1); break;
    case 2: SD_ATTN_G(2); break;
    case 4: SD_ATTN_G(4); break;
    default: SD_ATTN_G(8); break;
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
