// CATS down projection over the kept channels only (gfx950, wave64).
//
// "Sensitivity-Aware Thresholding and Token Routing for Activation
// Sparsification in Large Language Models" keeps the CATS runtime rule: only
// the channels whose post-gate activation survives the threshold contribute,
// so only their down-projection columns are read.  Here the down projection is
// stored transposed, w_down_t [d_ff, d], so one kept channel is one contiguous
// row of d elements.
//
// Grid: (column tiles) x (channel ranges).  A workgroup
//   1. compacts the kept channels of its range into an ascending LDS list with
//      a wave ballot + popcount prefix (the keep bytes come from the gate
//      kernel),
//   2. streams its column tile of each kept row (one 16-byte load per lane,
//      four rows in flight per lane) and accumulates hmid_i * w_down_t[i],
//   3. writes a partial sum for (range, tile); the last workgroup to finish a
//      tile (device-scope counter) adds the partials of all ranges in range
//      order, so the result is deterministic, and writes y (or y += result).
// Column-tile workgroups of range r also emit that range's part of the global
// ascending kept list at offset popcount(keep[0 .. range start)).
#include "common.hpp"
#include "internal.hpp"

namespace sd {

constexpr int kDownThreads = 256;
constexpr int kDownWaves = kDownThreads / kWave;

template <typename WT, int LPR>
__global__ __launch_bounds__(kDownThreads) void down_kernel(
    const WT* __restrict__ Wd, int d, int dff, const uint8_t* __restrict__ keep,
    const float* __restrict__ hmid, int range_len, int n_ranges, float* __restrict__ partials,
    unsigned* __restrict__ counters, float* __restrict__ y, int accumulate,
    int32_t* __restrict__ idx_out, int32_t* __restrict__ n_kept_out) {
  constexpr int RPW = kWave / LPR;        // row slots per wave
  constexpr int SLOTS = kDownWaves * RPW; // row slots per workgroup
  constexpr int TILE = 8 * LPR;           // columns per tile
  constexpr int U = 4;                    // rows in flight per slot
  extern __shared__ int list[];           // [range_len]
  __shared__ float red[kDownWaves][TILE];
  __shared__ int cnt_s, last_s, prefix_s;

  const int tile = blockIdx.x, range = blockIdx.y;
  const int i0 = range * range_len;
  const int i1 = min(dff, i0 + range_len);
  const int lane = lane_id(), wave = threadIdx.x / kWave;

  if (wave == 0) {
    int cnt = 0;
    for (int base = i0; base < i1; base += kWave) {
      const int i = base + lane;
      const bool f = i < i1 && keep[i] != 0;
      const unsigned long long m = __ballot(f);
      if (f) list[cnt + __popcll(m & ((1ull << lane) - 1ull))] = i;
      cnt += __popcll(m);
    }
    if (lane == 0) cnt_s = cnt;
  }
  __syncthreads();
  const int cnt = cnt_s;

  const int slot = wave * RPW + lane / LPR;
  const int col = tile * TILE + 8 * (lane % LPR);
  const bool col_ok = col < d;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int j = slot; j < cnt; j += U * SLOTS) {
    Vec8<WT> w[U];
    float hv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j + u * SLOTS;
      hv[u] = 0.f;
      if (jj < cnt && col_ok) {
        const int i = list[jj];
        hv[u] = hmid[i];
        w[u].load(Wd + (size_t)i * d + col);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j + u * SLOTS < cnt && col_ok) {
        float f[8];
        w[u].to_float(f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(hv[u], f[e], acc[e]);
      }
    }
  }
  // row slots of a wave -> one sum per column chunk (lanes 0..LPR-1)
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off);
  if (lane < LPR)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][8 * lane + e] = acc[e];
  __syncthreads();
  for (int c = threadIdx.x; c < TILE; c += kDownThreads) {
    const int gc = tile * TILE + c;
    if (gc < d) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kDownWaves; ++w) s += red[w][c];
      partials[(size_t)range * d + gc] = s;
    }
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) last_s = atomicAdd(&counters[tile], 1u) == (unsigned)(n_ranges - 1);
  __syncthreads();
  if (last_s) {
    __threadfence();
    for (int c = threadIdx.x; c < TILE; c += kDownThreads) {
      const int gc = tile * TILE + c;
      if (gc < d) {
        float s = 0.f;
        for (int r = 0; r < n_ranges; ++r) s += __builtin_nontemporal_load(partials + (size_t)r * d + gc);
        y[gc] = accumulate ? y[gc] + s : s;
      }
    }
  }

  if (idx_out && tile == 0) {
    int c = 0;
    for (int i = threadIdx.x; i < i0; i += kDownThreads) c += keep[i] != 0;
    c = (int)wave_sum((float)c);  // exact: counts stay far below 2^24
    if (threadIdx.x == 0) prefix_s = 0;
    __syncthreads();
    if (lane == 0) atomicAdd(&prefix_s, c);
    __syncthreads();
    const int prefix = prefix_s;
    for (int j = threadIdx.x; j < cnt; j += kDownThreads) idx_out[prefix + j] = list[j];
    if (range == n_ranges - 1 && threadIdx.x == 0) *n_kept_out = prefix + cnt;
  }
}

template <typename WT>
static void down_typed(const DownArgs& a, hipStream_t s) {
  dim3 grid(a.n_tiles, a.n_ranges);
  size_t lds = (size_t)a.range_len * sizeof(int);
  const WT* w = (const WT*)a.w_down_t;
  ProfScope prof(K_DOWN, s);
  switch (a.tile_cols) {
    case 128:
      down_kernel<WT, 16><<<grid, kDownThreads, lds, s>>>(w, a.d, a.dff, a.keep, a.hmid,
          a.range_len, a.n_ranges, a.partials, a.counters, a.y, a.accumulate, a.idx_out, a.n_kept_out);
      break;
    case 256:
      down_kernel<WT, 32><<<grid, kDownThreads, lds, s>>>(w, a.d, a.dff, a.keep, a.hmid,
          a.range_len, a.n_ranges, a.partials, a.counters, a.y, a.accumulate, a.idx_out, a.n_kept_out);
      break;
    default:
      down_kernel<WT, 64><<<grid, kDownThreads, lds, s>>>(w, a.d, a.dff, a.keep, a.hmid,
          a.range_len, a.n_ranges, a.partials, a.counters, a.y, a.accumulate, a.idx_out, a.n_kept_out);
      break;
  }
}

void launch_down(const DownArgs& a, int w_dtype, hipStream_t s) {
  if (w_dtype == 1) down_typed<bf16_t>(a, s);
  else down_typed<float>(a, s);
}

}  // namespace sd
