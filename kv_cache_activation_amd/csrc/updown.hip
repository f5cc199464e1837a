// CATS up and down projections over the kept channels only (gfx950, wave64).
//
// "Sensitivity-Aware Thresholding and Token Routing for Activation
// Sparsification in Large Language Models" keeps the CATS runtime rule: only
// the channels whose post-gate activation survives the threshold contribute,
// so only their up-projection rows and down-projection columns are read.  The
// down projection is stored transposed, w_down_t [d_ff, d], so a kept channel
// is one contiguous row of each matrix.
//
// The gate kernel has already written act and the keep bytes.  The kept
// channels, in ascending order, are dealt out to the P workgroups of this
// kernel in equal contiguous slices of the kept list (slice w = ranks
// [w n_k / P, (w + 1) n_k / P)), so every workgroup streams the same number of
// rows whatever the mask looks like.  A workgroup
//   1. counts the keep bytes of the whole d_ff range (one 64-byte chunk per
//      thread) and takes an exclusive block scan, which gives every kept
//      channel its rank; the channels of its slice go to an LDS list and,
//      with their ranks, to the global ascending index list;
//   2. issues the first group of its down rows (they depend only on the list),
//   3. computes u_j = W_up[c_j] . RMSNorm(h) for its channels, up to four
//      rows per wave with all their loads issued together, and
//      hmid_j = a_j u_j into LDS;
//   4. streams the down rows: wave v owns the 8-column chunks v*64 + lane (+
//      8*64 k) of every row, sixteen rows in flight per group with the next
//      group's loads issued before the current group's arithmetic, so the
//      accumulation y_w[c] = sum_j hmid_j w_down_t[c_j][c] needs no
//      cross-wave reduction;
//   5. writes its partial sum y_w [d].
// A second launch adds the P partials of each column in a fixed order and
// writes y (or y += result): deterministic, and the launch boundary makes the
// partials visible to every XCD, which on MI355X costs less than a hand-off
// inside one launch.
#include "common.hpp"
#include "internal.hpp"

namespace sd {

constexpr int kUdThreads = 512;
constexpr int kUdWaves = kUdThreads / kWave;
constexpr int kUdScanBytes = 64;  // keep bytes per thread: d_ff <= 64 * 512
constexpr int kRedCols = 16;      // reduce: columns per workgroup
constexpr int kRedSlices = 16;    // reduce: partition slices per column
constexpr int kRedPer = kUdMaxParts / kRedSlices;  // partitions per slice, at most

// Non-zero bytes of a 32-bit word as 4 bits (bit b = byte b != 0).
__device__ __forceinline__ uint32_t nz_bits(uint32_t w) {
  const uint32_t hi = (((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u;
  return ((hi >> 7) & 1u) | ((hi >> 14) & 2u) | ((hi >> 21) & 4u) | ((hi >> 28) & 8u);
}

template <typename WT, int NCH>
__global__ __launch_bounds__(kUdThreads) void up_down_kernel(
    const float* __restrict__ xin, const float* __restrict__ nw, float eps, int norm,
    const WT* __restrict__ Wu, const WT* __restrict__ Wd, int d, int dff, int chunk,
    const uint8_t* __restrict__ keep, const float* __restrict__ act, float* __restrict__ partials,
    int32_t* __restrict__ idx_out, int32_t* __restrict__ n_kept_out) {
  constexpr int U = 32 / (int)sizeof(WT);  // down rows per group (16 for bf16, 8 for fp32)
  __shared__ int list[kUdList];
  __shared__ float hm[kUdList];
  __shared__ int wave_tot[kUdWaves];
  extern __shared__ float xs[];
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int d8 = d >> 3;

  // 1. keep bytes [c0, c0 + chunk) of this thread, as a bit mask
  const int c0 = threadIdx.x * chunk;
  uint32_t kw[kUdScanBytes / 4];
#pragma unroll
  for (int q = 0; q < kUdScanBytes / 16; ++q) {
    const int off = c0 + 16 * q;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (16 * q < chunk) {
      if (off + 16 <= dff) {
        v = *reinterpret_cast<const uint4*>(keep + off);
      } else if (off < dff) {
        uint32_t b[4] = {0u, 0u, 0u, 0u};
        for (int e = 0; off + e < dff && e < 16; ++e) b[e >> 2] |= (uint32_t)keep[off + e] << (8 * (e & 3));
        v = make_uint4(b[0], b[1], b[2], b[3]);
      }
    }
    kw[4 * q] = v.x; kw[4 * q + 1] = v.y; kw[4 * q + 2] = v.z; kw[4 * q + 3] = v.w;
  }
  const float rs = stage_x<kUdThreads>(xin, norm ? nw : nullptr, d, eps, norm != 0, xs);
  uint64_t mask = 0;
#pragma unroll
  for (int q = 0; q < kUdScanBytes / 4; ++q) mask |= (uint64_t)nz_bits(kw[q]) << (4 * q);
  const int cnt = __popcll(mask);
  // exclusive block scan of cnt in thread order
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int before = incl - cnt, n_k = 0;
#pragma unroll
  for (int v = 0; v < kUdWaves; ++v) {
    before += v < wave ? wave_tot[v] : 0;
    n_k += wave_tot[v];
  }
  const int P = gridDim.x;
  const int lo = (int)((int64_t)blockIdx.x * n_k / P);
  const int hi = (int)((int64_t)(blockIdx.x + 1) * n_k / P);
  if (before < hi && before + cnt > lo) {
    uint64_t bits = mask;
    for (int r = before; bits; ++r) {
      const int bit = __ffsll((unsigned long long)bits) - 1;
      bits &= bits - 1;
      if (r >= lo && r < hi) {
        const int c = c0 + bit;
        list[r - lo] = c;
        if (idx_out) idx_out[r] = c;
      }
    }
  }
  if (n_kept_out && blockIdx.x == 0 && threadIdx.x == 0) *n_kept_out = n_k;
  __syncthreads();
  const int m = hi - lo;  // <= kUdList (the host sizes P so)

  // 2. first down group of this wave's first column chunk
  auto load_group = [&](Vec8<WT> (&w)[U], int j0, int c8) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (j0 + u < m) w[u].load(Wd + (size_t)list[j0 + u] * d + 8 * c8);
  };
  auto use_group = [&](const Vec8<WT> (&w)[U], int j0, float (&acc)[8]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + u < m) {
        const float h = hm[j0 + u];
        float f[8];
        w[u].to_float(f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(h, f[e], acc[e]);
      }
    }
  };
  const int c8_first = wave * kWave + lane;
  Vec8<WT> ga[U], gb[U];
  if (c8_first < d8) load_group(ga, 0, c8_first);

  // 3. up rows: hmid_j = a_j * (W_up[c_j] . x) * rs for this wave's list
  //    entries wave, wave + 8, ..., in batches whose loads are all issued
  //    before the first dot product (one wait per batch)
  {
    constexpr int kRowBytes = NCH * 8 * (int)sizeof(WT);  // per lane
    constexpr int B = kRowBytes >= 512 ? 1 : kRowBytes >= 256 ? 2 : 4;
#pragma unroll 1
    for (int j0 = wave; j0 < m; j0 += B * kUdWaves) {
      Row<WT, NCH> r[B];
      float av[B];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int j = j0 + b * kUdWaves;
        if (j < m) {
          if (d8 == NCH * kWave) r[b].load_full(Wu, d, list[j]);
          else r[b].load(Wu, d, list[j], d8);
        }
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int j = j0 + b * kUdWaves;
        av[b] = j < m ? act[list[j]] : 0.f;
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int j = j0 + b * kUdWaves;
        if (j < m) {
          const float u = r[b].dot(xs, d8) * rs;
          if (lane == 0) hm[j] = av[b] * u;
        }
      }
    }
  }
  __syncthreads();

  // 4. down rows, column chunk by column chunk
  for (int c8 = c8_first; c8 < d8; c8 += kUdWaves * kWave) {
    if (c8 != c8_first) load_group(ga, 0, c8);
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    int j0 = 0;
    while (j0 < m) {
      const int j1 = j0 + U;
      if (j1 < m) load_group(gb, j1, c8);
      use_group(ga, j0, acc);
      if (j1 >= m) break;
      const int j2 = j1 + U;
      if (j2 < m) load_group(ga, j2, c8);
      use_group(gb, j1, acc);
      j0 = j2;
    }
    // 5. this workgroup's partial sum
    store8(partials + (size_t)blockIdx.x * d + 8 * c8, acc);
  }
}

// y[c] (+)= sum over partitions w of partials[w][c]: slice s of a column sums
// partitions [s*per, s*per + per) in order, then the slices are added in order.
__global__ __launch_bounds__(kRedCols * kRedSlices) void mlp_reduce_kernel(
    const float* __restrict__ partials, int d, int P, float* __restrict__ y, int accumulate) {
  __shared__ float red[kRedSlices][kRedCols];
  const int cl = threadIdx.x % kRedCols, sl = threadIdx.x / kRedCols;
  const int c = blockIdx.x * kRedCols + cl;
  const int per = (P + kRedSlices - 1) / kRedSlices;
  const int w0 = sl * per;
  float v[kRedPer];
#pragma unroll
  for (int i = 0; i < kRedPer; ++i)
    v[i] = (c < d && i < per && w0 + i < P) ? partials[(size_t)(w0 + i) * d + c] : 0.f;
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kRedPer; ++i)
    if (i < per && w0 + i < P) sum += v[i];
  red[sl][cl] = sum;
  __syncthreads();
  if (sl == 0 && c < d) {
    float t = 0.f;
#pragma unroll
    for (int s = 0; s < kRedSlices; ++s) t += red[s][cl];
    y[c] = accumulate ? y[c] + t : t;
  }
}

int up_down_parts(int dff) {
  int p = (dff + kUdList - 1) / kUdList;
  return p < kUdMinParts ? kUdMinParts : p;
}

template <typename WT>
static void up_down_typed(const UpDownArgs& a, hipStream_t s) {
  const int P = up_down_parts(a.dff);
  int chunk = (a.dff + kUdThreads - 1) / kUdThreads;
  chunk = (chunk + 15) / 16 * 16;
  const size_t lds = (size_t)a.d * sizeof(float);
  SD_NCH_DISPATCH(a.d, launch_kernel(K_UP_DOWN, up_down_kernel<WT, NCH>, dim3(P),
                                     dim3(kUdThreads), (uint32_t)lds, s, a.x, a.norm, a.eps,
                                     (int)(a.norm != nullptr), (const WT*)a.w_up,
                                     (const WT*)a.w_down_t, a.d, a.dff, chunk, a.keep,
                                     (const float*)a.act, a.partials, a.idx_out, a.n_kept_out));
  launch_kernel(K_MLP_REDUCE, mlp_reduce_kernel, dim3((a.d + kRedCols - 1) / kRedCols),
                dim3(kRedCols * kRedSlices), 0, s, (const float*)a.partials, a.d, P, a.y,
                a.accumulate);
}

void launch_up_down(const UpDownArgs& a, int w_dtype, hipStream_t s) {
  if (w_dtype == 1) up_down_typed<bf16_t>(a, s);
  else up_down_typed<float>(a, s);
}

}  // namespace sd
