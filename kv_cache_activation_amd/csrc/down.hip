// CATS down projection over the kept channels only (gfx950, wave64).
//
// "Sensitivity-Aware Thresholding and Token Routing for Activation
// Sparsification in Large Language Models" keeps the CATS runtime rule: only
// the channels whose post-gate activation survives the threshold contribute,
// so only their down-projection columns are read.  The down projection is
// stored transposed, w_down_t [d_ff, d], so a kept channel is one contiguous
// row.
//
// The gate kernel has already written the keep bytes and hmid_i = a_i u_i for
// the kept channels.  The kept channels, in ascending order, are dealt out to
// the P workgroups of this kernel in equal contiguous slices of the kept list
// (slice w = ranks [w n_k / P, (w + 1) n_k / P)), so every workgroup streams
// the same number of rows whatever the mask looks like.  A workgroup
//   1. counts the keep bytes of the whole d_ff range (one 64-byte chunk per
//      thread) and takes an exclusive block scan, which gives every kept
//      channel its rank; the channels of its slice go to an LDS list and,
//      with their ranks, to the global ascending index list;
//   2. streams the down rows: wave v owns the 8-column chunks v*64 + lane (+
//      8*64 k) of every row, lane j holds hmid of list entry j, and a batch
//      of 32 rows (16 for float32 weights) is in flight at once -- a whole
//      slice at 50% sparsity -- so the accumulation
//      y_w[c] = sum_j hmid_j w_down_t[c_j][c] needs no cross-wave reduction;
//   3. writes its partial sum y_w [d].
// A second launch adds the P partials of each column in a fixed order and
// writes y (or y += result): deterministic, and the launch boundary makes the
// partials visible to every XCD, which on MI355X costs less than a hand-off
// inside one launch.
//
// Batches: with nb sequences sharing the weight reads ("Where Activation
// Sparsity and KV-Cache Sparsity Cross in LLM Decoding", §3.3 "Dispatch and
// batching") the keep bytes are the union of the batch's masks, hmid is
// [nb, d_ff] (zero where a sequence dropped a channel the union keeps), each
// row read once serves all nb sequences, and the partials are [P, nb, d].
#include "common.hpp"
#include "internal.hpp"

namespace sd {

constexpr int kDownThreads = 512;
constexpr int kDownWaves = kDownThreads / kWave;
constexpr int kDownScanBytes = 64;  // keep bytes per thread: d_ff <= 64 * 512
constexpr int kRedCols = 32;      // reduce: columns per workgroup (128-byte pieces of a partial)
constexpr int kRedSlices = 16;    // reduce: partition slices per column
constexpr int kRedPer = kDownMaxParts / kRedSlices;  // partitions per slice, at most

// Non-zero bytes of a 32-bit word as 4 bits (bit b = byte b != 0).
__device__ __forceinline__ uint32_t nz_bits(uint32_t w) {
  const uint32_t hi = (((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u;
  return ((hi >> 7) & 1u) | ((hi >> 14) & 2u) | ((hi >> 21) & 4u) | ((hi >> 28) & 8u);
}

template <typename WT, int NB>
__global__ __launch_bounds__(kDownThreads) void down_kernel(
    const WT* __restrict__ Wd, int d, int dff, int chunk, const uint8_t* __restrict__ keep,
    const float* __restrict__ hmid, int nb, float* __restrict__ partials,
    int32_t* __restrict__ idx_out, int32_t* __restrict__ n_kept_out) {
  // rows per batch: 32 for bf16, 16 for fp32, halved for four or more sequences
  constexpr int U = 64 / (int)sizeof(WT) / (NB >= 4 ? 2 : 1);
  __shared__ int list[kDownList];
  __shared__ int wave_tot[kDownWaves];
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int d8 = d >> 3;

  // 1. keep bytes [c0, c0 + chunk) of this thread, as a bit mask
  const int c0 = threadIdx.x * chunk;
  uint32_t kw[kDownScanBytes / 4];
#pragma unroll
  for (int q = 0; q < kDownScanBytes / 16; ++q) {
    const int off = c0 + 16 * q;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (16 * q < chunk) {
      if (off + 16 <= dff) {
        v = *reinterpret_cast<const uint4*>(keep + off);
      } else if (off < dff) {
        uint32_t b[4] = {0u, 0u, 0u, 0u};
        for (int e = 0; off + e < dff && e < 16; ++e)
          b[e >> 2] |= (uint32_t)keep[off + e] << (8 * (e & 3));
        v = make_uint4(b[0], b[1], b[2], b[3]);
      }
    }
    kw[4 * q] = v.x; kw[4 * q + 1] = v.y; kw[4 * q + 2] = v.z; kw[4 * q + 3] = v.w;
  }
  uint64_t mask = 0;
#pragma unroll
  for (int q = 0; q < kDownScanBytes / 4; ++q) mask |= (uint64_t)nz_bits(kw[q]) << (4 * q);
  const int cnt = __popcll(mask);
  // exclusive block scan of cnt in thread order
  const int incl = wave_incl_scan(cnt);
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int before = incl - cnt, n_k = 0;
#pragma unroll
  for (int v = 0; v < kDownWaves; ++v) {
    before += v < wave ? wave_tot[v] : 0;
    n_k += wave_tot[v];
  }
  const int P = gridDim.x;
  const int lo = (int)((int64_t)blockIdx.x * n_k / P);
  const int hi = (int)((int64_t)(blockIdx.x + 1) * n_k / P);
  // the slice's channels: each thread that holds part of it hands its mask to
  // its whole wave (lane b takes bit b, ranked by a popcount), so a list entry
  // costs one step instead of one iteration of a serial walk over the bits
  uint64_t holders = __ballot(before < hi && before + cnt > lo);  // wave-uniform
  while (holders) {
    const int src = __ffsll((unsigned long long)holders) - 1;
    holders &= holders - 1;
    const uint32_t mlo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mask, src);
    const uint32_t mhi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mask >> 32), src);
    const uint64_t mk = ((uint64_t)mhi << 32) | mlo;
    const int bf = __builtin_amdgcn_readlane(before, src);
    if ((mk >> lane) & 1ull) {
      const int r = bf + __popcll(mk & ((1ull << lane) - 1ull));
      if (r >= lo && r < hi) {
        const int c = (wave * kWave + src) * chunk + lane;
        list[r - lo] = c;
        if (idx_out) idx_out[r] = c;
      }
    }
  }
  if (n_kept_out && blockIdx.x == 0 && threadIdx.x == 0) *n_kept_out = n_k;
  __syncthreads();
  const int m = hi - lo;  // <= kDownList = 64 (the host sizes P so)

  // 2. lane j holds hmid of list entry j.  The rows go in batches of U, all
  //    of a batch's loads issued back to back with no branch between them:
  //    entries past the slice's end repeat its last channel (a repeat of a
  //    line already requested, served by the cache) with weight 0, so the
  //    compiler can let each row's FMAs wait for that row alone.
  if (m == 0) {  // wave-uniform: an empty slice still writes its zero partial
    for (int c8 = wave * kWave + lane; c8 < d8; c8 += kDownWaves * kWave) {
      const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int b = 0; b < nb; ++b) store8(partials + ((size_t)blockIdx.x * nb + b) * d + 8 * c8, z);
    }
    return;
  }
  float hv[NB];  // hmid of list entry `lane`, per sequence
#pragma unroll
  for (int b = 0; b < NB; ++b)
    hv[b] = lane < m && b < nb ? hmid[(size_t)b * dff + list[lane]] : 0.f;
  for (int c8 = wave * kWave + lane; c8 < d8; c8 += kDownWaves * kWave) {
    float acc[NB][8];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[b][e] = 0.f;
#pragma unroll 1
    for (int j0 = 0; j0 < m; j0 += U) {
      Vec8<WT> g[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = min(j0 + u, m - 1);
        g[u].load(Wd + (size_t)list[j] * d + 8 * c8);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float f[8];
        g[u].to_float(f);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float hj =
              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hv[b]), j0 + u));
          const float h = j0 + u < m ? hj : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[b][e] = fmaf(h, f[e], acc[b][e]);
        }
      }
    }
    // 3. this workgroup's partial sums
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (b < nb) store8(partials + ((size_t)blockIdx.x * nb + b) * d + 8 * c8, acc[b]);
  }
}

// y[c] (+)= sum over partitions w of partials[w][c]: slice s of a column sums
// partitions [s*per, s*per + per) in order, then the slices are added in order.
// A workgroup's 32 columns make each partial read one 128-byte piece (16
// columns read half lines, which HBM counters show as twice the bytes).
__global__ __launch_bounds__(kRedCols * kRedSlices) void mlp_reduce_kernel(
    const float* __restrict__ partials, int d, int P, float* __restrict__ y, int accumulate) {
  __shared__ float red[kRedSlices][kRedCols];
  const int cl = threadIdx.x % kRedCols, sl = threadIdx.x / kRedCols;
  const int c = blockIdx.x * kRedCols + cl;
  // the value accumulated into, read with the partials rather than after them
  const float y_old = accumulate && sl == 0 && c < d ? y[c] : 0.f;
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
    y[c] = y_old + t;
  }
}

int down_parts(int dff) {
  int p = (dff + kDownList - 1) / kDownList;
  return p < kDownMinParts ? kDownMinParts : p;
}

template <typename WT>
static void down_typed(const DownArgs& a, hipStream_t s) {
  const int P = down_parts(a.dff);
  int chunk = (a.dff + kDownThreads - 1) / kDownThreads;
  chunk = (chunk + 15) / 16 * 16;
  const int nb = a.nb > 1 ? a.nb : 1;
#define SD_DOWN(NBV)                                                                        \
  launch_kernel(K_DOWN, down_kernel<WT, NBV>, dim3(P), dim3(kDownThreads), 0, s,            \
                (const WT*)a.w_down_t, a.d, a.dff, chunk, a.keep, a.hmid, nb, a.partials,   \
                a.idx_out, a.n_kept_out)
  if (nb == 1) SD_DOWN(1);
  else if (nb == 2) SD_DOWN(2);
  else if (nb <= 4) SD_DOWN(4);
  else SD_DOWN(8);
#undef SD_DOWN
  // the partials [P, nb, d] are [P, nb d]: one reduce over nb d columns
  const int cols = nb * a.d;
  launch_kernel(K_MLP_REDUCE, mlp_reduce_kernel, dim3((cols + kRedCols - 1) / kRedCols),
                dim3(kRedCols * kRedSlices), 0, s, (const float*)a.partials, cols, P, a.y,
                a.accumulate);
}

void launch_down(const DownArgs& a, int w_dtype, hipStream_t s) {
  if (w_dtype == 1) down_typed<bf16_t>(a, s);
  else down_typed<float>(a, s);
}

}  // namespace sd
