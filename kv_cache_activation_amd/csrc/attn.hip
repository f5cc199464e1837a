// Split-K GQA decode attention (gfx950, wave64).
//
// "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding"
// reads every cache -- full in dense mode, gathered in KV mode -- through one
// split-K decoding kernel (§1, §4.1), and §4.4 shows why the dense baseline
// must be that efficient path.  This is this library's own design for CDNA:
//
//   one launch, grid (splits, KV heads): a workgroup owns a contiguous chunk
//   of rows of one KV head and serves all G query heads of the group, so each
//   K/V byte is read once.  A row of d_h elements is spread over d_h/16 lanes
//   (two 16-byte loads per lane, each load instruction covering whole 128-byte
//   lines); the wave holds 64/(d_h/16) row slots, and two register buffers of
//   U rows per slot alternate, so the next rows are in flight while the
//   current ones are computed (the chunk is read in address order).  The
//   kernel spends its vector-ALU time on the dot products and the P V update:
//   wide rows per lane keep the lane exchanges and the softmax bookkeeping
//   per element small, and the running maximum is only raised (with a
//   rescale) when a logit passes it by 2^8.
//   Every lane group keeps its own online-softmax state (max, sum, acc) in the
//   log2 domain; at the end the groups write their states to LDS and the
//   workgroup merges them into one (m, l, acc[d_h]) per query head and split.
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
// Lazy rescaling: the running maximum of a lane group only moves when a new
// logit exceeds it by more than this (log2 domain), so the exponentials stay
// below 2^8 and the accumulator is rescaled a few times per chunk, not per row.
constexpr float kLazyMax = 8.f;
// Maximum of a lane group that has seen no row yet: finite, so 2^(z - m) of a
// masked logit (z = -inf) is 0 and never NaN.
constexpr float kNoRow = -1e30f;
// Register buffers of rows in rotation (NBUF - 1 in flight during a compute):
// three for chunks of at least kAttnLongChunk rows (one cache and one length;
// measured at 131072 rows per head, 4096-row chunks: dense decoding 5178-5180
// -> 5148-5161 us per step), two otherwise (three slowed the 410-row chunks of
// the KV branch at 131072 and the batched chunks).
constexpr int kAttnBufs = 2;
constexpr int kAttnLongChunk = 2048;

// Max and sum over aligned groups of N lanes (16, 32 or 64), VALU exchanges.
template <int N>
__device__ __forceinline__ float slot_max(float x) {
  static_assert(N == 16 || N == 32 || N == 64, "slot groups of 16, 32 or 64 lanes");
  x = group_max<16>(x);
  if (N >= 32) x = fmaxf(x, xor_lanes<16>(x));
  if (N >= 64) x = fmaxf(x, xor_lanes<32>(x));
  return x;
}
template <int N>
__device__ __forceinline__ float slot_sum(float x) {
  static_assert(N == 16 || N == 32 || N == 64, "slot groups of 16, 32 or 64 lanes");
  x = group_sum<16>(x);
  if (N >= 32) x += xor_lanes<16>(x);
  if (N >= 64) x += xor_lanes<32>(x);
  return x;
}

// Raw v_exp_f32: 2^x with -inf -> 0.  The arguments here are at most kLazyMax,
// and results that would be denormal only lose weights below 2^-126.
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

// Split-K partial attention.  EPL = elements of a row per lane (16, or 8 when
// G = 8 so that the query and accumulator registers fit): a row of d_h
// elements is spread over LPR = d_h / EPL lanes, lane `sub` holding the
// 8-element pieces at 8 sub + h d_h / H for h < H = EPL / 8, so each 16-byte
// load instruction of the wave covers whole 128-byte lines of its rows.  A
// dot product then needs log2(LPR) lane exchanges per query head (3 for
// d_h = 128), and the softmax bookkeeping is shared by EPL elements.
// Two register buffers of U rows per slot alternate: the loads of the next
// U * SLOTS rows are in flight while the current ones are computed.  Rows
// past the chunk's end load the chunk's last row (a repeat the cache serves)
// and get weight 0.
// MODE: 0 = one cache and one length (grid (splits, groups)); 1 = ragged
// per-head lengths; 2 = a batch of sequences.  A compile-time mode leaves the
// plain path without the branches that would make it fetch its arguments in
// several dependent rounds.
template <typename KT, int DH, int G, int U, int EPL, int MODE, int NBUF>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(
    const float* __restrict__ q, const KT* __restrict__ K, const KT* __restrict__ V, int cap,
    int n_ctx, int sink, int shift, int kv_div, int ragged, HeadInts lens, HeadInts starts,
    int batched, AttnBatch bt, int h_q, float scale_log2, int chunk, int n_splits,
    float* __restrict__ pm, float* __restrict__ pl, float* __restrict__ pacc) {
  constexpr int H = EPL / 8;           // 8-element pieces per lane and row
  constexpr int LPR = DH / EPL;        // lanes per row
  constexpr int RPW = kWave / LPR;     // row slots per wave
  constexpr int SLOTS = kAttnWaves * RPW;
  constexpr int STEP = U * SLOTS;      // rows of one register buffer
  static_assert(LPR == 4 || LPR == 8 || LPR == 16, "lanes per row");
  // per row slot: its softmax state; 64 KB of LDS at most (SLOTS G DH floats)
  __shared__ float sm_m[SLOTS][G], sm_l[SLOTS][G], sm_M[G], sm_L[G];
  __shared__ __align__(16) float sm_w[G][SLOTS];
  __shared__ __align__(16) float sm_acc[SLOTS][G][DH];

  // grid (splits, groups); ragged: a flat grid, block b belongs to the last
  // head whose first chunk starts at or before b (starts ascending, unused
  // entries past the last head hold INT_MAX)
  int split = blockIdx.x, kv = blockIdx.y;
  if constexpr (MODE == 1) {
    kv = 0;
#pragma unroll
    for (int h = 1; h < kMaxKvHeads; ++h) kv += (int)(split >= starts.v[h]);
    split -= starts.v[kv];
  }
  // batched: a flat grid over (sequence, KV head, chunk); each sequence reads
  // its own cache with its own query rows and partial slots
  int seq = 0, rows = n_ctx;
  if constexpr (MODE == 1) rows = lens.v[(kv / kv_div) & (kMaxKvHeads - 1)];
  if constexpr (MODE == 2) {
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
  // pointers in registers now: one round of argument loads, not one per branch
  asm volatile("" ::"s"(q), "s"(K), "s"(V), "s"(pm), "s"(pl), "s"(pacc));
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

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNoRow;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  if (r0 < r1) {  // workgroup-uniform; every chunk of a launch holds rows
    Vec8<KT> kbuf[NBUF][U][H], vbuf[NBUF][U][H];
    // rows jb + slot + u SLOTS of this lane, clamped into the chunk
    auto issue = [&](Vec8<KT>(&kr)[U][H], Vec8<KT>(&vr)[U][H], int jb) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t o = phys(min(jb + slot + u * SLOTS, r1 - 1)) * DH;
#pragma unroll
        for (int h = 0; h < H; ++h) {
          kr[u][h].load(Kb + o + h * (DH / H));
          vr[u][h].load(Vb + o + h * (DH / H));
        }
      }
    };
    // the first NBUF - 1 buffers in flight before the query is read
#pragma unroll
    for (int i = 0; i + 1 < NBUF; ++i) issue(kbuf[i], vbuf[i], r0 + i * STEP);

    float qv[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int h = 0; h < H; ++h) {
        float t[8];
        load8f(q + (size_t)(kv * G + g) * DH + 8 * sub + h * (DH / H), t);
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[g][8 * h + e] = t[e] * scale_log2;
      }
    }

    auto compute = [&](const Vec8<KT>(&kr)[U][H], const Vec8<KT>(&vr)[U][H], int jb) {
      float p[U][G];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float kf[EPL];
#pragma unroll
        for (int h = 0; h < H; ++h) {
          float t[8];
          kr[u][h].to_float(t);
#pragma unroll
          for (int e = 0; e < 8; ++e) kf[8 * h + e] = t[e];
        }
        const bool ok = jb + slot + u * SLOTS < r1;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float t = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) t = fmaf(kf[e], qv[g][e], t);
          t = group_sum<LPR>(t);
          p[u][g] = ok ? t : -INFINITY;
        }
      }
      float mb[G];
      bool up = false;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        mb[g] = p[0][g];
#pragma unroll
        for (int u = 1; u < U; ++u) mb[g] = fmaxf(mb[g], p[u][g]);
        up |= mb[g] > m[g] + kLazyMax;
      }
      if (up) {  // per lane; after the first rows of a chunk this is rare
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float mn = fmaxf(m[g], mb[g]);
          const float alpha = exp2_raw(m[g] - mn);
          l[g] *= alpha;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
          m[g] = mn;
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          p[u][g] = exp2_raw(p[u][g] - m[g]);
          l[g] += p[u][g];
        }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float vf[EPL];
#pragma unroll
        for (int h = 0; h < H; ++h) {
          float t[8];
          vr[u][h].to_float(t);
#pragma unroll
          for (int e = 0; e < 8; ++e) vf[8 * h + e] = t[e];
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p[u][g], vf[e], acc[g][e]);
      }
    };

    // NBUF buffers in rotation: step k of a round issues iteration it + k +
    // NBUF - 1 into the buffer freed by step k - 1, then computes iteration
    // it + k, so NBUF - 1 buffers of rows are in flight during every compute.
    // The issues are unconditional (past the end they repeat row r1 - 1, one
    // line per lane group that the cache serves), so every wait for a buffer
    // counts exactly the newer buffers' loads as still in flight; the
    // scheduling barriers keep each buffer's loads together ahead of the
    // arithmetic.
    const int n_it = (r1 - r0 + STEP - 1) / STEP;  // >= 1, uniform
    for (int it = 0; it < n_it; it += NBUF) {
#pragma unroll
      for (int k = 0; k < NBUF; ++k) {
        issue(kbuf[(k + NBUF - 1) % NBUF], vbuf[(k + NBUF - 1) % NBUF],
              r0 + (it + k + NBUF - 1) * STEP);
        __builtin_amdgcn_sched_barrier(0);
        if (k == 0 || it + k < n_it) compute(kbuf[k], vbuf[k], r0 + (it + k) * STEP);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // Merge of the workgroup's row slots through LDS: each lane group writes its
  // state once, lane reductions turn the slot maxima into weights 2^(m_slot -
  // M), then every thread sums two columns over the slots.  (A tree of lane exchanges costs about a thousand
  // vector instructions per lane for 4 heads x 16 elements, more than a short
  // chunk's whole stream.)
  if (sub == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sm_m[slot][g] = m[g];
      sm_l[slot][g] = l[g];
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int h = 0; h < H; ++h) {
      float* dst = &sm_acc[slot][g][8 * sub + h * (DH / H)];
      reinterpret_cast<float4*>(dst)[0] =
          make_float4(acc[g][8 * h], acc[g][8 * h + 1], acc[g][8 * h + 2], acc[g][8 * h + 3]);
      reinterpret_cast<float4*>(dst)[1] =
          make_float4(acc[g][8 * h + 4], acc[g][8 * h + 5], acc[g][8 * h + 6], acc[g][8 * h + 7]);
    }
  __syncthreads();
  // slot weights: lane group g of SLOTS threads holds slot s = t % SLOTS of
  // head g; lane reductions give M_g = max_s m_s and L_g = sum_s l_s 2^(m_s - M_g)
  {
    const int t = threadIdx.x;
    if (t < G * SLOTS) {  // whole lane groups
      const int g = t / SLOTS, s2 = t - g * SLOTS;
      const float ms = sm_m[s2][g];
      const float M = slot_max<SLOTS>(ms);
      const float w = exp2_raw(ms - M);
      const float L = slot_sum<SLOTS>(sm_l[s2][g] * w);
      sm_w[g][s2] = w;
      if (s2 == 0) {
        sm_M[g] = M;
        sm_L[g] = L;
      }
    }
  }
  __syncthreads();
  // outputs: two adjacent columns of one head per thread, four slot weights
  // per LDS read
  for (int o = threadIdx.x; o < G * DH / 2; o += kAttnThreads) {
    const int g = o / (DH / 2), c = 2 * (o - g * (DH / 2));
    float A0 = 0.f, A1 = 0.f;
#pragma unroll
    for (int s4 = 0; s4 < SLOTS; s4 += 4) {
      const float4 w4 = *reinterpret_cast<const float4*>(&sm_w[g][s4]);
      const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float2 a = *reinterpret_cast<const float2*>(&sm_acc[s4 + k][g][c]);
        A0 = fmaf(a.x, wv[k], A0);
        A1 = fmaf(a.y, wv[k], A1);
      }
    }
    const size_t hs = ((size_t)seq * h_q + kv * G + g) * n_splits + split;
    *reinterpret_cast<float2*>(pacc + hs * DH + c) = make_float2(A0, A1);
    if (c == 0) {
      const float L = sm_L[g];
      pm[hs] = L > 0.f ? sm_M[g] : -INFINITY;  // a split without rows: (-inf, 0, 0)
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

template <int DH, int CAP, int MODE>
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
  asm volatile("" ::"s"(pm), "s"(pl), "s"(pacc), "s"(out), "s"(lse));  // one round of argument loads
  int ns = stride;  // MODE as in attn_kernel
  if constexpr (MODE == 1) ns = counts.v[(h / G) & (kMaxKvHeads - 1)];
  if constexpr (MODE == 2) ns = bt.splits[(h / h_q) & 7];
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
#define SD_ATTN_M(GG, UU, EE, MM, NB)                                                       \
  launch_kernel(K_ATTN_PARTIAL, attn_kernel<KT, DH, GG, UU, EE, MM, NB>, grid,                   \
                dim3(kAttnThreads), 0,                                                        \
                s, a.q, k, v, a.cap, a.n_ctx, a.sink, a.shift, kv_div, a.ragged, a.lens, starts,   \
                a.batched, a.bt, a.h_q, scale_log2, a.chunk, a.n_splits, a.pm, a.pl, a.pacc)
#define SD_ATTN_G(GG, UU, EE)                                       \
  do {                                                              \
    if (a.batched) SD_ATTN_M(GG, UU, EE, 2, kAttnBufs);             \
    else if (a.ragged) SD_ATTN_M(GG, UU, EE, 1, kAttnBufs);         \
    else if (a.chunk >= kAttnLongChunk) SD_ATTN_M(GG, UU, EE, 0, 3); \
    else SD_ATTN_M(GG, UU, EE, 0, kAttnBufs);                       \
  } while (0)
  switch (G) {
    // rows per slot and buffer: one for four query heads per KV head (measured
    // on MI355X with one workgroup per CU: 13114 rows 16.8 us with one, 17.3
    // with two, 18.1 with three)
    case 1: SD_ATTN_G(1, 2, 16); break;
    case 2: SD_ATTN_G(2, 2, 16); break;
    case 4: SD_ATTN_G(4, 1, 16); break;
    default: SD_ATTN_G(8, 1, 8); break;
  }
#undef SD_ATTN_G
#undef SD_ATTN_M
  if (a.no_merge) return;  // the consumer merges the partials itself
  const dim3 mgrid(nq, DH / kMergeCols);
  const int G_all = a.h_q / a.h_kv;
#define SD_MERGE_M(CAPV, MM)                                                                   \
  launch_kernel(K_ATTN_COMBINE, attn_merge_kernel<DH, CAPV, MM>, mgrid, dim3(kMergeThreads), 0, s, \
                a.pm, a.pl, a.pacc, a.n_splits, a.ragged, counts, G_all, a.batched, a.bt, a.h_q,   \
                a.out, a.lse)
#define SD_MERGE(CAPV)                        \
  do {                                        \
    if (a.batched) SD_MERGE_M(CAPV, 2);       \
    else if (a.ragged) SD_MERGE_M(CAPV, 1);   \
    else SD_MERGE_M(CAPV, 0);                 \
  } while (0)
  if (a.n_splits <= 32) SD_MERGE(32);
  else if (a.n_splits <= 64) SD_MERGE(64);
  else if (a.n_splits <= 128) SD_MERGE(128);
  else SD_MERGE(kMaxSplits);
#undef SD_MERGE
#undef SD_MERGE_M
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
