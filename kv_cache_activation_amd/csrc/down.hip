// CATS down projection over the kept channels only (gfx950, wave64).
//
// "Sensitivity-Aware Thresholding and Token Routing for Activation
// Sparsification in Large Language Models" keeps the CATS runtime rule: only
// the channels whose post-gate activation survives the threshold contribute,
// so only their down-projection columns are read.  Here the down projection is
// stored transposed, w_down_t [d_ff, d], so one kept channel is one contiguous
// row of d elements.
//
// Grid: (512-column tiles) x (channel ranges).  A workgroup
//   1. compacts the kept channels of its range into an ascending LDS list with
//      wave ballots and popcount prefixes (the keep bytes and the hmid values
//      of the range come from the gate kernel, loaded in one round),
//   2. streams the 1 KB segment (one 16-byte load per lane) of each kept row
//      that falls in its tile, in groups of sixteen rows per wave with the
//      next group's loads issued before the current group's arithmetic,
//      accumulating hmid_i * w_down_t[i],
//   3. writes a partial sum for (range, tile).
// A second launch adds the partials of all ranges in range order --
// deterministic -- and writes y (or y += result): one thread per column, every
// range's value loaded before the first is used.  The launch boundary makes
// the partials visible to every XCD, which on MI355X costs less than a
// hand-off inside one launch.
// Column-tile-0 workgroups of range r also emit that range's part of the
// global ascending kept list at offset popcount(keep[0 .. range start)).
#include "common.hpp"
#include "internal.hpp"

namespace sd {

constexpr int kDownThreads = 256;
constexpr int kDownWaves = kDownThreads / kWave;
constexpr int kDownTile = 512;   // columns per tile: 64 lanes x 8 columns
constexpr int kDownRounds = 2;   // range_len <= 512 = kDownRounds * kDownThreads
constexpr int kDownMaxRanges = 64;  // channel ranges per call (the tail sum holds them in VGPRs)

// Block-wide exclusive prefix count of `flag` in thread order, and the total.
__device__ __forceinline__ int down_prefix(bool flag, int* wave_tot, int& total) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const unsigned long long m = __ballot(flag);
  if (lane == 0) wave_tot[wave] = __popcll(m);
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int v = 0; v < kDownWaves; ++v) {
    before += v < wave ? wave_tot[v] : 0;
    total += wave_tot[v];
  }
  __syncthreads();
  return before + __popcll(m & ((1ull << lane) - 1ull));
}

template <typename WT>
__global__ __launch_bounds__(kDownThreads) void down_kernel(
    const WT* __restrict__ Wd, int d, int dff, const uint8_t* __restrict__ keep,
    const float* __restrict__ hmid, int range_len, int n_ranges, float* __restrict__ partials,
    int32_t* __restrict__ idx_out, int32_t* __restrict__ n_kept_out) {
  constexpr int U = 16;  // rows per group; two groups in flight per wave
  __shared__ int list[kDownRounds * kDownThreads];
  __shared__ float hv_s[kDownRounds * kDownThreads];
  __shared__ float red[kDownWaves][kDownTile];
  __shared__ int wave_tot[kDownWaves];
  __shared__ int prefix_s;

  const int tile = blockIdx.x, range = blockIdx.y;
  const int i0 = range * range_len;
  const int i1 = min(dff, i0 + range_len);
  const int lane = lane_id(), wave = threadIdx.x / kWave;

  // ascending list of the kept channels of [i0, i1), with their hmid values
  // (hmid of a dropped channel is stale and never used)
  bool f[kDownRounds];
  float hv[kDownRounds];
#pragma unroll
  for (int r = 0; r < kDownRounds; ++r) {
    const int i = i0 + r * kDownThreads + threadIdx.x;
    f[r] = false;
    hv[r] = 0.f;
    if (i < i1) {
      f[r] = keep[i] != 0;
      hv[r] = hmid[i];
    }
  }
  int cnt = 0;
#pragma unroll
  for (int r = 0; r < kDownRounds; ++r) {
    if (i0 + r * kDownThreads >= i1) break;
    int tot;
    const int pos = cnt + down_prefix(f[r], wave_tot, tot);
    if (f[r]) {
      list[pos] = i0 + r * kDownThreads + threadIdx.x;
      hv_s[pos] = hv[r];
    }
    cnt += tot;
  }
  __syncthreads();

  const int col = tile * kDownTile + 8 * lane;
  const bool col_ok = col < d;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  // rows j0 + u*kDownWaves (u < U) form a group of this wave
  auto load_group = [&](Vec8<WT> (&w)[U], int j0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j0 + u * kDownWaves;
      if (jj < cnt && col_ok) w[u].load(Wd + (size_t)list[jj] * d + col);
    }
  };
  auto use_group = [&](const Vec8<WT> (&w)[U], int j0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j0 + u * kDownWaves;
      if (jj < cnt && col_ok) {
        const float h = hv_s[jj];
        float fw[8];
        w[u].to_float(fw);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(h, fw[e], acc[e]);
      }
    }
  };
  constexpr int STEP = U * kDownWaves;
  Vec8<WT> wa[U], wb[U];
  int j0 = wave;
  if (j0 < cnt) load_group(wa, j0);
  while (j0 < cnt) {
    const int j1 = j0 + STEP;
    if (j1 < cnt) load_group(wb, j1);
    use_group(wa, j0);
    if (j1 >= cnt) break;
    const int j2 = j1 + STEP;
    if (j2 < cnt) load_group(wa, j2);
    use_group(wb, j1);
    j0 = j2;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[wave][8 * lane + e] = acc[e];
  __syncthreads();
  for (int c = threadIdx.x; c < kDownTile; c += kDownThreads) {
    const int gc = tile * kDownTile + c;
    if (gc < d) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kDownWaves; ++w) sum += red[w][c];
      partials[(size_t)range * d + gc] = sum;
    }
  }

  if (idx_out && tile == 0) {
    // offset of this range's list: kept channels before i0 (bytes are 0 or 1)
    int c = 0;
    const uint32_t* kw = reinterpret_cast<const uint32_t*>(keep);
    for (int q = threadIdx.x; q < i0 / 4; q += kDownThreads) c += (int)((kw[q] * 0x01010101u) >> 24);
    c = wave_sum_int(c);
    if (threadIdx.x == 0) prefix_s = 0;
    __syncthreads();
    if (lane == 0) atomicAdd(&prefix_s, c);
    __syncthreads();
    const int prefix = prefix_s;
    for (int j = threadIdx.x; j < cnt; j += kDownThreads) idx_out[prefix + j] = list[j];
    if (range == n_ranges - 1 && threadIdx.x == 0) *n_kept_out = prefix + cnt;
  }
}

// y[c] (+)= sum over ranges r, in order, of partials[r][c]
__global__ __launch_bounds__(256) void down_reduce_kernel(const float* __restrict__ partials,
                                                          int d, int n_ranges,
                                                          float* __restrict__ y, int accumulate) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  float v[kDownMaxRanges];
#pragma unroll
  for (int r = 0; r < kDownMaxRanges; ++r)
    v[r] = (c < d && r < n_ranges) ? partials[(size_t)r * d + c] : 0.f;
  if (c >= d) return;
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < kDownMaxRanges; ++r)
    if (r < n_ranges) sum += v[r];
  y[c] = accumulate ? y[c] + sum : sum;
}

template <typename WT>
static void down_typed(const DownArgs& a, hipStream_t s) {
  dim3 grid(a.n_tiles, a.n_ranges);
  launch_kernel(K_DOWN, down_kernel<WT>, grid, dim3(kDownThreads), 0, s, (const WT*)a.w_down_t,
                a.d, a.dff, a.keep, a.hmid, a.range_len, a.n_ranges, a.partials, a.idx_out,
                a.n_kept_out);
  launch_kernel(K_DOWN_REDUCE, down_reduce_kernel, dim3((a.d + 255) / 256), dim3(256), 0, s,
                (const float*)a.partials, a.d, a.n_ranges, a.y, a.accumulate);
}

void launch_down(const DownArgs& a, int w_dtype, hipStream_t s) {
  if (w_dtype == 1) down_typed<bf16_t>(a, s);
  else down_typed<float>(a, s);
}

}  // namespace sd
