// TEAL-style sparse projections: column-gathered GEMV over the kept input
// channels (gfx950, wave64).
//
// "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding"
// takes its projection branch from TEAL (§3.2 "Sparse Branches", §4.1
// "Setup"): each of a layer's seven projections keeps only the input
// channels whose magnitude clears a calibrated threshold and loads only those
// channels' weights.  With the weight stored transposed, w_t [d_in, d_out],
// a kept input channel j is one contiguous row, and
//     y = sum over kept j of x_j w_t[j]
// reads exactly the kept rows.
//
// One launch, grid (P slices, column tiles of 4096 outputs, or 1024 with
// four row groups for a narrow single matrix whose slices leave compute
// units idle).  A workgroup
//   1. reads the whole input vector (one chunk per thread), applies the
//      RMSNorm when given (x * rs * norm_w, rs reduced over the workgroup),
//      decides keep_j = |x_j| > t (t < 0: all) in float32, and takes an
//      exclusive block scan of the per-thread counts, which ranks every kept
//      channel; the ranks [s n_k / P, (s + 1) n_k / P) form its slice, so
//      every workgroup reads the same number of rows whatever the mask;
//   2. streams its slice's rows over its column tile: wave v owns the
//      8-column chunks of 512 columns, lane j holds x of list entry j, and a
//      batch of rows is loaded with no branch between the loads (entries
//      past the slice repeat its last row with weight 0);
//   3. writes a partial sum [d_out] per slice.  With two weight matrices
//      (gate and up share their input) it does both.
// A second launch adds the P partials of each column in a fixed order and
// applies the projection's epilogue: plain (y = or +=), SwiGLU
// (hmid = SiLU(gate) * up), or the QKV epilogue (RoPE on q and k, q out,
// k and v rounded and appended to the caches).  Deterministic.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace sd {

constexpr int kTealThreads = 512;
constexpr int kTealWaves = kTealThreads / kWave;
constexpr int kTealTile = kTealWaves * kWave * 8;  // 4096 output columns per workgroup
constexpr int kRCols = 16, kRSlices = 16;          // QKV reduce: 16 columns x 16 slices
constexpr int kRCols2 = 32;  // plain reduce: 32 columns, so a partial is read in 128-byte pieces
constexpr int kRPer = kTealMaxParts / kRSlices;    // partitions per slice, at most

// NQ float4 chunks of the input per thread (d_in <= 4 NQ 512).
// RG row groups: the workgroup's column tile is kTealTile / RG columns and
// its eight waves form RG groups that take interleaved rows of the slice;
// the groups' sums are added in LDS in a fixed order.  RG > 1 gives narrow
// projections (O, QKV) more workgroups at the same slice count, so the
// partial sums do not grow.
template <typename WT, int NQ, bool DUAL, int RG>
__global__ __launch_bounds__(kTealThreads) void teal_kernel(
    const float* __restrict__ x, int d_in, const float* __restrict__ nw, float eps, float t,
    const WT* __restrict__ W0, const WT* __restrict__ W1, int d_out,
    float* __restrict__ part0, float* __restrict__ part1, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ n_kept_out, uint8_t* __restrict__ keep_out) {
  constexpr int U = (DUAL ? 32 : 64) / (int)sizeof(WT) / RG;  // rows per batch, matrix and group
  constexpr int CW = kTealWaves / RG;                          // waves per row group
  constexpr int TILE = kTealTile / RG;                         // output columns per workgroup
  __shared__ int list[kTealList];
  __shared__ float xl[kTealList];
  __shared__ int wave_tot[kTealWaves];
  __shared__ float red[kTealWaves];
  const int lane = lane_id(), wave = threadIdx.x / kWave;

  // 1. this thread's inputs [c0, c0 + 4 NQ)
  const int c0 = threadIdx.x * 4 * NQ;
  float4 xv[NQ];
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int i = c0 + 4 * q;
    xv[q] = i < d_in ? *reinterpret_cast<const float4*>(x + i) : make_float4(0.f, 0.f, 0.f, 0.f);
    ss = fmaf(xv[q].x, xv[q].x, fmaf(xv[q].y, xv[q].y, fmaf(xv[q].z, xv[q].z, fmaf(xv[q].w, xv[q].w, ss))));
  }
  if (nw) {  // RMSNorm: x * rs * nw
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int v = 0; v < kTealWaves; ++v) tot += red[v];
    const float rs = 1.0f / sqrtf(tot / (float)d_in + eps);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int i = c0 + 4 * q;
      if (i < d_in) {
        const float4 w = *reinterpret_cast<const float4*>(nw + i);
        xv[q] = make_float4(xv[q].x * rs * w.x, xv[q].y * rs * w.y, xv[q].z * rs * w.z,
                            xv[q].w * rs * w.w);
      }
    }
  }
  uint64_t mask = 0;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const float e[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (c0 + 4 * q + k < d_in && (t < 0.f || fabsf(e[k]) > t)) mask |= 1ull << (4 * q + k);
  }
  if (keep_out && blockIdx.x == 0 && blockIdx.y == 0) {
#pragma unroll
    for (int b = 0; b < 4 * NQ; ++b)
      if (c0 + b < d_in) keep_out[c0 + b] = (uint8_t)((mask >> b) & 1ull);
  }
  const int cnt = __popcll(mask);
  const int incl = wave_incl_scan(cnt);
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int before = incl - cnt, n_k = 0;
#pragma unroll
  for (int v = 0; v < kTealWaves; ++v) {
    before += v < wave ? wave_tot[v] : 0;
    n_k += wave_tot[v];
  }
  const int P = gridDim.x, s = blockIdx.x;
  const int lo = (int)((int64_t)s * n_k / P);
  const int hi = (int)((int64_t)(s + 1) * n_k / P);
  if (before < hi && before + cnt > lo) {  // this thread holds part of the slice
    int r = before;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const float e[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if ((mask >> (4 * q + k)) & 1ull) {
          if (r >= lo && r < hi) {
            list[r - lo] = c0 + 4 * q + k;
            xl[r - lo] = e[k];
            if (idx_out && blockIdx.y == 0) idx_out[r] = c0 + 4 * q + k;
          }
          ++r;
        }
      }
    }
  }
  if (n_kept_out && s == 0 && blockIdx.y == 0 && threadIdx.x == 0) *n_kept_out = n_k;
  __syncthreads();
  const int m = hi - lo;  // <= kTealList (the host sizes P so)

  // 2. rows of the slice over this workgroup's column tile; row group rg
  //    takes list entries rg, rg + RG, ...
  const int rg = __builtin_amdgcn_readfirstlane(wave / CW), cw = wave - rg * CW;
  const int d8 = d_out >> 3;
  const int c8 = blockIdx.y * (TILE / 8) + cw * kWave + lane;
  const bool col_ok = c8 < d8;
  const float hv = lane < m ? xl[lane] : 0.f;
  float acc0[8], acc1[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc0[e] = acc1[e] = 0.f;
  if (m > 0 && col_ok) {
#pragma unroll 1
    for (int j0 = rg; j0 < m; j0 += U * RG) {
      Vec8<WT> g0[U], g1[DUAL ? U : 1];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t row = (size_t)list[min(j0 + RG * u, m - 1)] * d_out + 8 * c8;
        g0[u].load(W0 + row);
        if constexpr (DUAL) g1[u].load(W1 + row);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + RG * u;  // wave-uniform
        const float hj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hv), min(j, 63)));
        const float h = j < m ? hj : 0.f;
        float f[8];
        g0[u].to_float(f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc0[e] = fmaf(h, f[e], acc0[e]);
        if constexpr (DUAL) {
          g1[DUAL ? u : 0].to_float(f);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc1[e] = fmaf(h, f[e], acc1[e]);
        }
      }
    }
  }
  if constexpr (RG > 1) {  // row groups 1.. add into group 0, in order
    __shared__ float grp[kTealWaves * kWave * 8];  // 16 KB
    static_assert(!DUAL, "row groups are for single-matrix projections");
    if (rg > 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) grp[((wave - CW) * kWave + lane) * 8 + e] = acc0[e];
    }
    __syncthreads();
    if (rg == 0) {
#pragma unroll
      for (int r = 1; r < RG; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc0[e] += grp[(((r - 1) * CW + cw) * kWave + lane) * 8 + e];
    }
  }
  // 3. partial sums of this slice
  if (rg == 0 && col_ok) {
    store8(part0 + (size_t)s * d_out + 8 * c8, acc0);
    if constexpr (DUAL) store8(part1 + (size_t)s * d_out + 8 * c8, acc1);
  }
}

// Sum of the P partials of column c: slice sl of the column sums partitions
// [sl per, sl per + per) in order, then the slices are added in order.
template <int COLS>
__device__ __forceinline__ float column_sum(const float* __restrict__ part, int P, int d_out,
                                            int c, int sl, int cl, float (*red)[COLS]) {
  const int per = (P + kRSlices - 1) / kRSlices;
  const int w0 = sl * per;
  float v[kRPer];
#pragma unroll
  for (int i = 0; i < kRPer; ++i)
    v[i] = (c < d_out && i < per && w0 + i < P) ? part[(size_t)(w0 + i) * d_out + c] : 0.f;
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kRPer; ++i)
    if (i < per && w0 + i < P) sum += v[i];
  red[sl][cl] = sum;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int k = 0; k < kRSlices; ++k) tot += red[k][cl];
  return tot;
}

// y[c] (+)= sum of partials (EPI 0), or y[c] = SiLU(sum part0) * (sum part1) (EPI 1).
// keep (optional): keep[c] = |y[c]| > t (t < 0: 1), decided on the float32
// value stored, the rule the next projection applies to its input.
template <int EPI>
__global__ __launch_bounds__(kRCols2 * kRSlices) void teal_reduce_kernel(
    const float* __restrict__ part0, const float* __restrict__ part1, int P, int d_out,
    float* __restrict__ y, int accumulate, float t, uint8_t* __restrict__ keep) {
  __shared__ float red0[kRSlices][kRCols2], red1[kRSlices][kRCols2];
  const int cl = threadIdx.x % kRCols2, sl = threadIdx.x / kRCols2;
  const int c = blockIdx.x * kRCols2 + cl;
  const float a = column_sum<kRCols2>(part0, P, d_out, c, sl, cl, red0);
  float b = 0.f;
  if (EPI == 1) b = column_sum<kRCols2>(part1, P, d_out, c, sl, cl, red1);
  if (sl == 0 && c < d_out) {
    const float v = EPI == 1 ? silu(a) * b : accumulate ? y[c] + a : a;
    y[c] = v;
    if (keep) keep[c] = t < 0.f || fabsf(v) > t;
  }
}

// QKV epilogue: a workgroup owns 8 rotation pairs (i, i + d_h/2) of one head:
// columns head d_h + i0 .. +8 and head d_h + d_h/2 + i0 .. +8 (d_h/2 % 8 == 0).
template <typename KT>
__global__ __launch_bounds__(kRCols * kRSlices) void teal_qkv_reduce_kernel(
    const float* __restrict__ part, int P, int d_out, int h_q, int h_kv, int dh,
    RopeTable rope, float* __restrict__ q_out, KT* __restrict__ k_full, KT* __restrict__ v_full,
    int cap_full, int row_full, KT* __restrict__ k_sel, KT* __restrict__ v_sel, int cap_sel,
    int row_sel, int ragged, HeadInts sel_rows) {
  __shared__ float red[kRSlices][kRCols];
  __shared__ float tot[kRCols];
  const int half = dh >> 1;
  const int per_head = half / 8;  // workgroups per head
  const int head = blockIdx.x / per_head, i0 = (blockIdx.x % per_head) * 8;
  const int cl = threadIdx.x % kRCols, sl = threadIdx.x / kRCols;
  const int c = head * dh + (cl < 8 ? i0 + cl : half + i0 + cl - 8);
  const float v = column_sum<kRCols>(part, P, d_out, c, sl, cl, red);
  if (sl == 0) tot[cl] = v;
  __syncthreads();
  if (threadIdx.x >= 8) return;
  const int i = i0 + threadIdx.x;
  float a = tot[threadIdx.x], b = tot[threadIdx.x + 8];
  if (head < h_q + h_kv) {  // rotate q and k, not v
    const float cs = rope.c[i], sn = rope.s[i];
    const float ra = a * cs - b * sn, rb = b * cs + a * sn;
    a = ra;
    b = rb;
  }
  if (head < h_q) {
    q_out[head * dh + i] = a;
    q_out[head * dh + i + half] = b;
  } else {
    const bool is_k = head < h_q + h_kv;
    const int kv = is_k ? head - h_q : head - h_q - h_kv;
    KT* full = is_k ? k_full : v_full;
    const size_t off = ((size_t)kv * cap_full + row_full) * dh + i;
    store_elem(full + off, a);
    store_elem(full + off + half, b);
    if (k_sel) {
      KT* sel = is_k ? k_sel : v_sel;
      // ragged budgets: each KV head appends at its own row
      const int rsel = ragged ? sel_rows.v[kv & (kMaxKvHeads - 1)] : row_sel;
      const size_t offs = ((size_t)kv * cap_sel + rsel) * dh + i;
      store_elem(sel + offs, a);
      store_elem(sel + offs + half, b);
    }
  }
}

TealGrid teal_grid(int d_in, int d_out) {
  TealGrid g;
  g.tiles = (d_out + kTealTile - 1) / kTealTile;
  int p = kTealMinBlocks / g.tiles;
  const int need = (d_in + kTealList - 1) / kTealList;
  if (p < need) p = need;
  if (p < 1) p = 1;
  g.parts = p;
  return g;
}

// Row groups for a projection: four for a single matrix of at most 8192
// outputs whose slices and tiles fill at most half the compute units (O and
// QKV of the 8B-class layer: 256 and 384 workgroups at 64 slices instead of
// 64 and 128), one otherwise.  Measured on MI355X: the down projection (224
// slices of a 14336-wide input) went from 20.6 to 25.7 us per launch with
// four groups, its rows read in 2 KB pieces with no idle units to gain.
template <bool DUAL>
static int teal_row_groups(const TealGrid& g, int d_out) {
  return !DUAL && d_out <= 8192 && 2 * g.parts * g.tiles <= cu_count_dev() ? 4 : 1;
}

template <typename WT, bool DUAL>
static void teal_typed(const TealArgs& a, hipStream_t s) {
  const TealGrid g = teal_grid(a.d_in, a.d_out);  // slices as the workspace is sized
  const int rgs = teal_row_groups<DUAL>(g, a.d_out);
  const int tiles = (a.d_out + kTealTile / rgs - 1) / (kTealTile / rgs);
  const int nq4 = (a.d_in + 4 * kTealThreads - 1) / (4 * kTealThreads);  // float4 per thread
#define SD_TEAL(NQ, RGV)                                                                    \
  launch_kernel(a.kind, teal_kernel<WT, NQ, DUAL, RGV>, dim3(g.parts, tiles),                \
                dim3(kTealThreads), 0, s, a.x, a.d_in, a.norm, a.eps, a.t, (const WT*)a.w0,   \
                (const WT*)a.w1, a.d_out, a.part0, a.part1, a.idx_out, a.n_kept_out,          \
                a.keep_out)
#define SD_TEAL_RG(NQ)           \
  do {                           \
    if constexpr (!DUAL) {       \
      if (rgs == 4) {            \
        SD_TEAL(NQ, 4);          \
        break;                   \
      }                          \
    }                            \
    SD_TEAL(NQ, 1);              \
  } while (0)
  if (nq4 <= 2) SD_TEAL_RG(2);
  else if (nq4 <= 4) SD_TEAL_RG(4);
  else if (nq4 <= 8) SD_TEAL_RG(8);
  else SD_TEAL_RG(16);
#undef SD_TEAL_RG
#undef SD_TEAL
}

void launch_teal(const TealArgs& a, int w_dtype, hipStream_t s) {
  const bool dual = a.w1 != nullptr;
  if (w_dtype == 1) {
    if (dual) teal_typed<bf16_t, true>(a, s);
    else teal_typed<bf16_t, false>(a, s);
  } else {
    if (dual) teal_typed<float, true>(a, s);
    else teal_typed<float, false>(a, s);
  }
}

void launch_teal_reduce(const float* part0, const float* part1, int parts, int d_out, float* y,
                        int accumulate, int swiglu, int kind, hipStream_t s, float t,
                        uint8_t* keep) {
  const dim3 grid((d_out + kRCols2 - 1) / kRCols2), block(kRCols2 * kRSlices);
  if (swiglu)
    launch_kernel(kind, teal_reduce_kernel<1>, grid, block, 0, s, part0, part1, parts, d_out, y,
                  accumulate, t, keep);
  else
    launch_kernel(kind, teal_reduce_kernel<0>, grid, block, 0, s, part0, part1, parts, d_out, y,
                  accumulate, t, keep);
}

void launch_teal_qkv_reduce(const float* part, int parts, const QkvArgs& a, int kv_dtype,
                            hipStream_t s) {
  const int d_out = (a.h_q + 2 * a.h_kv) * a.dh;
  const dim3 grid((a.h_q + 2 * a.h_kv) * (a.dh / 2 / 8)), block(kRCols * kRSlices);
#define SD_QKV_R(KT)                                                                          \
  launch_kernel(K_TEAL_QKV_REDUCE, teal_qkv_reduce_kernel<KT>, grid, block, 0, s, part, parts, \
                d_out, a.h_q, a.h_kv, a.dh, a.rope, a.q_out, (KT*)a.k_full, (KT*)a.v_full,     \
                a.cap_full, a.row_full, (KT*)a.k_sel, (KT*)a.v_sel, a.cap_sel, a.row_sel,       \
                a.ragged, a.sel_rows)
  if (kv_dtype == 1) SD_QKV_R(bf16_t);
  else SD_QKV_R(float);
#undef SD_QKV_R
}

}  // namespace sd
