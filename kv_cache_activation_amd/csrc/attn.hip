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
//   Ragged per-head lengths launch only the chunks that hold rows: a flat
//   grid whose block index is mapped to (KV head, chunk) by per-head prefix
//   counts, so a few long heads next to many short ones leave no idle
//   workgroups behind.
//
//   A second, small launch merges the splits: workgroup (query head, 32
//   columns), eight split groups of 32 threads; every thread loads its share
//   of split values at once (one memory round trip), the workgroup turns the
//   split maxima into weights meanwhile,
//   out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s, lse = (M + log2 L) ln 2,
//   and the groups are added in a fixed order, so the result does not depend
//   on scheduling.  The launch
//   boundary makes the partials visible to every XCD; measured on MI355X it is
//   cheaper than a hand-off inside one launch (coherent stores, a wait for
//   their acknowledgement, a ticket and coherent loads are three memory round
//   trips).
#include <limits.h>
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace sd {

constexpr int kAttnThreads = 256;
constexpr int kMaxSplits = 256;  // splits per KV head (the merge holds a column's share in VGPRs)
constexpr int kAttnWaves = kAttnThreads / kWave;

template <typename KT, int DH, int G, int U>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(
    const float* __restrict__ q, const KT* __restrict__ K, const KT* __restrict__ V, int cap,
    int n_ctx, int sink, int shift, int kv_div, int ragged, HeadInts lens, HeadInts starts,
    int batched, AttnBatch bt, int h_q, float scale_log2, int chunk, int n_splits,
    float* __restrict__ pm, float* __restrict__ pl, float* __restrict__ pacc) {
  constexpr int LPR = DH / 8;          // lanes per row
  constexpr int RPW = kWave / LPR;     // row slots per wave
  constexpr int SLOTS = kAttnWaves * RPW;
  __shared__ float sm_m[kAttnWaves][G], sm_l[kAttnWaves][G];
  __shared__ float sm_acc[kAttnWaves][G][DH];

  // grid (splits, groups); ragged: a flat grid, block b belongs to the last
  // head whose first chunk starts at or before b (starts ascending, unused
  // entries past the last head hold INT_MAX)
  int split = blockIdx.x, kv = blockIdx.y;
  if (ragged) {
    kv = 0;
#pragma unroll
    for (int h = 1; h < kMaxKvHeads; ++h) kv += (int)(split >= starts.v[h]);
    split -= starts.v[kv];
  }
  // batched: a flat grid over (sequence, KV head, chunk); each sequence reads
  // its own cache with its own query rows and partial slots
  int seq = 0, rows = ragged ? lens.v[(kv / kv_div) & (kMaxKvHeads - 1)] : n_ctx;
  if (batched) {
#pragma unroll
    for (int b = 1; b < 8; ++b) seq += (int)(split >= bt.starts[b]);
    const int local = split - bt.starts[seq];
    kv = local / bt.splits[seq];
    split = local - kv * bt.splits[seq];
    K = (const KT*)bt.k[seq];
    V = (const KT*)bt.v[seq];
    cap = bt.cap[seq];
    chunk = bt.chunk[seq];
    rows = bt.rows[seq];
    q += (size_t)seq * h_q * DH;
  }
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int sub = lane % LPR;
  const int slot = wave * RPW + lane / LPR;
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
    const size_t hs = ((size_t)seq * h_q + kv * G + g) * n_splits + split;
    pacc[hs * DH + c] = A;
    if (c == 0) {
      pm[hs] = M;
      pl[hs] = L;
    }
  }
}

// Merge of the splits: workgroup (query head, kMergeCols columns); thread t
// serves column t % kMergeCols for splits g, g + kMergeGroups, ... (g = t /
// kMergeCols), at most CAP splits.  Loads come from clamped indices, so none
// depends on a branch and all are in flight together; splits past the count
// get weight zero.  Ragged lengths: query head h reads counts.v[h / G] splits;
// a batch: query head h of the flat [nb, h_q] list reads its sequence's count.
constexpr int kMergeThreads = 256;
constexpr int kMergeCols = 32;
constexpr int kMergeGroups = kMergeThreads / kMergeCols;

template <int DH, int CAP>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(
    const float* __restrict__ pm, const float* __restrict__ pl, const float* __restrict__ pacc,
    int stride, int ragged, HeadInts counts, int G, int batched, AttnBatch bt, int h_q,
    float* __restrict__ out, float* __restrict__ lse) {
  constexpr int PER = CAP / kMergeGroups;  // splits per thread
  constexpr int NW = kMergeThreads / kWave;
  __shared__ float w_s[CAP];
  __shared__ float red_m[NW], red_l[NW];
  __shared__ float share[kMergeGroups][kMergeCols];
  const int h = blockIdx.x, t = threadIdx.x;
  const int col = blockIdx.y * kMergeCols + t % kMergeCols, grp = t / kMergeCols;
  const int ns = batched  ? bt.splits[(h / h_q) & 7]
                 : ragged ? counts.v[(h / G) & (kMaxKvHeads - 1)]
                          : stride;
  const float* base = pacc + (size_t)h * stride * DH + col;
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int sp = min(grp + i * kMergeGroups, ns - 1);
    v[i] = base[(size_t)sp * DH];
  }
  // split weights: thread t owns split t (CAP <= kMergeThreads)
  const int ts = min(t, ns - 1);
  const float mt = t < ns ? pm[(size_t)h * stride + ts] : -INFINITY;
  const float lt = pl[(size_t)h * stride + ts];
  const int lane = lane_id(), wave = t / kWave;
  float M = wave_max(mt);
  if (lane == 0) red_m[wave] = M;
  __syncthreads();
  M = red_m[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, red_m[w]);
  const float wt = mt == -INFINITY ? 0.f : exp2f(mt - M);
  if (t < CAP) w_s[t] = wt;
  const float lsum = wave_sum(wt * (t < ns ? lt : 0.f));
  if (lane == 0) red_l[wave] = lsum;
  __syncthreads();
  float L = red_l[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) L += red_l[w];
  float A = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int sp = grp + i * kMergeGroups;
    if (sp < ns) A = fmaf(w_s[sp], v[i], A);
  }
  share[grp][t % kMergeCols] = A;
  __syncthreads();
  if (grp) return;
  float S = share[0][t];
#pragma unroll
  for (int g = 1; g < kMergeGroups; ++g) S += share[g][t];
  out[(size_t)h * DH + col] = S / L;
  if (lse && col == 0) lse[h] = (M + log2f(L)) * 0.69314718055994530942f;
}

template <typename KT, int DH>
static void attn_dh(const AttnArgs& a, hipStream_t s) {
  // per_query_head: one workgroup (group of one) per query head, reading KV head h / G
  const int G = a.per_query_head ? 1 : a.h_q / a.h_kv;
  const int kv_div = a.per_query_head ? a.h_q / a.h_kv : 1;
  const int groups = a.per_query_head ? a.h_q : a.h_kv;
  const float scale_log2 = a.scale * 1.44269504088896340736f;
  dim3 grid(a.n_splits, groups);
  // ragged: chunks per KV head and the flat grid's per-head first block
  HeadInts counts{}, starts{};
  if (a.ragged) {
    int total = 0;
    for (int h = 0; h < kMaxKvHeads; ++h) {
      counts.v[h] = h < a.h_kv ? (a.lens.v[h] + a.chunk - 1) / a.chunk : 0;
      starts.v[h] = h < a.h_kv ? total : INT_MAX;
      total += counts.v[h];
    }
    grid = dim3(total, 1);
  }
  int nq = a.h_q;  // query heads the merge covers
  if (a.batched) {
    int total = 0;
    for (int b = 0; b < a.batched; ++b) total += a.h_kv * a.bt.splits[b];
    grid = dim3(total, 1);
    nq = a.batched * a.h_q;
  }
  const KT* k = (const KT*)a.k;
  const KT* v = (const KT*)a.v;
#define SD_ATTN_G(GG, UU)                                                                   \
  launch_kernel(K_ATTN_PARTIAL, attn_kernel<KT, DH, GG, UU>, grid, dim3(kAttnThreads), 0, s, \
                a.q, k, v, a.cap, a.n_ctx, a.sink, a.shift, kv_div, a.ragged, a.lens, starts,        \
                a.batched, a.bt, a.h_q, scale_log2, a.chunk, a.n_splits, a.pm, a.pl, a.pacc)
  switch (G) {
    case 1: SD_ATTN_G(1, 8); break;
    case 2: SD_ATTN_G(2, 8); break;
    case 4: SD_ATTN_G(4, 4); break;
    default: SD_ATTN_G(8, 4); break;
  }
#undef SD_ATTN_G
  const dim3 mgrid(nq, DH / kMergeCols);
  const int G_all = a.h_q / a.h_kv;
#define SD_MERGE(CAPV)                                                                        \
  launch_kernel(K_ATTN_COMBINE, attn_merge_kernel<DH, CAPV>, mgrid, dim3(kMergeThreads), 0, s, \
                a.pm, a.pl, a.pacc, a.n_splits, a.ragged, counts, G_all, a.batched, a.bt, a.h_q, \
                a.out, a.lse)
  if (a.n_splits <= 64) SD_MERGE(64);
  else if (a.n_splits <= 128) SD_MERGE(128);
  else SD_MERGE(kMaxSplits);
#undef SD_MERGE
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
