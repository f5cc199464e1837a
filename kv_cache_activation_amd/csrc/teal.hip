// TEAL-style sparse projections over column blocks of the weight (gfx950,
// wave64).
//
// "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding"
// takes its projection branch from TEAL (§3.2 "Sparse Branches", §4.1
// "Setup"): each of a layer's seven projections keeps only the input
// channels whose magnitude clears a calibrated threshold and loads only those
// channels' weights, y = sum over kept j of x_j w[j, :].
//
// Layout.  The weight is stored in blocks of 128 output columns,
// w_blk [nblk][d_in][128]: within a block, input channel j is one contiguous
// 256-byte piece (bf16), and a block's rows are contiguous.  A workgroup that
// owns one block reads, for each kept channel, exactly that channel's piece:
// two whole 128-byte lines, with no other workgroup sharing them.
//
// Grid (S slices, nblk blocks), 512 threads.  Workgroup (s, b):
//   1. with an RMSNorm, adds up x^2 over the whole input (every workgroup
//      needs the scale); then decides keep_j = |x_j * rs * norm_j| > t (t < 0:
//      all) in float32 for the channels of its slice [s R, (s + 1) R) and
//      ranks the kept ones in channel order (block scan of per-thread counts);
//   2. streams the kept channels' pieces of block b: lane l loads 16 bytes of
//      row (l / 16) of a group of four, so a wave instruction brings four
//      rows and the eight waves thirty-two; U instructions per wave are issued
//      before any arithmetic, entries past the list's end repeat its last
//      row with weight 0;
//   3. adds its thirty-two row groups in LDS in a fixed order and stores the
//      slice's partial sums of the block with agent-scope stores (written
//      through to memory, where every XCD's loads see them), then takes a
//      ticket for the block;
//   4. the slice that draws the last ticket of the block adds the S partials
//      in slice order (agent-scope loads), clears the ticket for the next
//      launch, and applies the projection's epilogue to the block's columns:
//      y = or y +=; SwiGLU with the next projection's keep bytes; or RoPE on q
//      and k with q written out and k, v rounded and appended to the caches.
// No workgroup waits for another: the ones that do not finish last exit, and
// the last one finds every partial stored.  One launch per projection, and
// the summation order is fixed, so results do not depend on scheduling.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace sd {

// 512 threads: a compute unit holding two workgroups streams with sixteen
// waves (against 256 threads, measured at 8B-class widths with 50% kept:
// down 15.6 -> 15.2 us, O 9.5 -> 8.8-9.2, gate + up 25.9 -> 25.2-25.7, QKV
// unchanged)
constexpr int kTbThreads = 512;
constexpr int kTbWaves = kTbThreads / kWave;   // 8
constexpr int kTbSub = kWave / 16;             // rows per wave load instruction (4)
constexpr int kTbGroups = kTbWaves * kTbSub;   // row groups of a workgroup (32)
constexpr int kTbCh = kTealMaxRange / kTbThreads;  // slice channels per thread, at most (4)
static_assert(kTealBlock == 16 * 8, "a block row is 16 lanes x 8 columns");

template <typename WT, bool DUAL, int EPI, typename KT>
__global__ __launch_bounds__(kTbThreads) void teal_kernel(TealArgs a) {
  // rows per wave instruction group in flight: 8 instructions (32 rows) per
  // matrix and wave for bf16, half for float32
  constexpr bool ACC = EPI == TEAL_ACC || EPI == TEAL_DOWN || EPI == TEAL_CATS_DOWN;
  constexpr int U = (DUAL ? 8 : 16) * 2 / (int)sizeof(WT);
  __shared__ int list[kTealMaxRange];
  __shared__ float xl[kTealMaxRange];
  __shared__ int wave_tot[kTbWaves];
  __shared__ float wred[kTbWaves];
  __shared__ float red[kTbGroups][(DUAL ? 2 : 1) * kTealBlock];
  __shared__ float col[(DUAL ? 2 : 1) * kTealBlock];
  __shared__ unsigned tk_s;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int S = gridDim.x, s = blockIdx.x, b = blockIdx.y;
  const int d_in = a.d_in, d_out = a.d_out;
  const int nblk = gridDim.y;
  const float* __restrict__ x = a.x;
  const float* __restrict__ nw = a.norm;
  constexpr int NCOL = (DUAL ? 2 : 1) * kTealBlock;  // <= kTbThreads
  // y += : the block's current outputs, loaded with the inputs (only the
  // block's last slice writes them, at the end)
  float y_old = 0.f;
  if constexpr (ACC) {
    const int c = b * kTealBlock + threadIdx.x % kTealBlock;
    if (threadIdx.x < NCOL && c < d_out) y_old = (threadIdx.x >= kTealBlock ? a.y2 : a.y)[c];
  }

  // 1. this slice's inputs (and norm weights) are loaded with the pass that
  //    adds up x^2 for the RMSNorm scale, so both take one memory round trip
  const int R = (d_in + S - 1) / S;
  const int r0 = s * R, r1 = min(d_in, r0 + R);
  const int ch = (R + kTbThreads - 1) / kTbThreads;  // <= kTbCh
  const int c0 = r0 + threadIdx.x * ch;              // this thread's channels [c0, c0 + ch)
  float xv[kTbCh], wv[kTbCh];
#pragma unroll
  for (int k = 0; k < kTbCh; ++k) {
    const int c = min(c0 + k, d_in - 1);  // unconditional loads, discarded past the slice
    xv[k] = k < ch ? x[c] : 0.f;
    wv[k] = nw && k < ch ? nw[c] : 1.f;
  }
  float rs = 1.f;
  if (nw) {
    float ss = 0.f;
    for (int i = 4 * threadIdx.x; i < d_in; i += 4 * kTbThreads) {
      const float4 v = *reinterpret_cast<const float4*>(x + i);
      ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
    }
    ss = wave_sum(ss);
    if (lane == 0) wred[wave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int v = 0; v < kTbWaves; ++v) tot += wred[v];
    rs = 1.0f / sqrtf(tot / (float)d_in + a.eps);
  }
  uint32_t mask = 0;
#pragma unroll
  for (int k = 0; k < kTbCh; ++k) {
    float v = 0.f;
    if (k < ch && c0 + k < r1) {
      v = xv[k];
      if (nw) v = v * rs * wv[k];
      if (a.t < 0.f || fabsf(v) > a.t) mask |= 1u << k;
    }
    xv[k] = v;
  }
  if (a.keep_out && b == 0) {
#pragma unroll
    for (int k = 0; k < kTbCh; ++k)
      if (k < ch && c0 + k < r1) a.keep_out[c0 + k] = (uint8_t)((mask >> k) & 1u);
  }
  const int cnt = __popc(mask);
  const int incl = wave_incl_scan(cnt);
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int before = incl - cnt, m = 0;
#pragma unroll
  for (int v = 0; v < kTbWaves; ++v) {
    before += v < wave ? wave_tot[v] : 0;
    m += wave_tot[v];
  }
  {
    int r = before;
#pragma unroll
    for (int k = 0; k < kTbCh; ++k)
      if ((mask >> k) & 1u) {
        list[r] = c0 + k;
        xl[r] = xv[k];
        ++r;
      }
  }
  if ((a.idx_out || a.n_kept_out) && b == 0) {
    // ranks before this slice: the kept channels of [0, r0), same rule
    int prior = 0;
    for (int c = threadIdx.x; c < r0; c += kTbThreads) {
      float v = x[c];
      if (nw) v = v * rs * nw[c];
      prior += (a.t < 0.f || fabsf(v) > a.t) ? 1 : 0;
    }
    prior = (int)wave_sum((float)prior);  // exact below 2^24
    __syncthreads();
    if (lane == 0) wave_tot[wave] = prior;
    __syncthreads();
    int off = 0;
#pragma unroll
    for (int v = 0; v < kTbWaves; ++v) off += wave_tot[v];
    if (a.idx_out) {
      int r = before;
#pragma unroll
      for (int k = 0; k < kTbCh; ++k)
        if ((mask >> k) & 1u) a.idx_out[off + r++] = c0 + k;
    }
    if (a.n_kept_out && s == S - 1 && threadIdx.x == 0) *a.n_kept_out = off + m;
  }
  __syncthreads();

  // 2. the kept channels' pieces of block b; lane (sub, q): row sub of each
  //    group of four, columns 8q .. 8q + 7 of the block
  const int sub = lane >> 4, q = lane & 15;
  const WT* __restrict__ W0 = static_cast<const WT*>(a.w0) + (size_t)b * d_in * kTealBlock + 8 * q;
  const WT* __restrict__ W1 =
      DUAL ? static_cast<const WT*>(a.w1) + (size_t)b * d_in * kTealBlock + 8 * q : nullptr;
  float acc0[8], acc1[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc0[e] = acc1[e] = 0.f;
  const int g = wave * kTbSub + sub;  // this lane's row group
#pragma unroll 1
  for (int j0 = 0; j0 < m; j0 += U * kTbGroups) {
    Vec8<WT> w0[U], w1[DUAL ? U : 1];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = min(j0 + u * kTbGroups + g, m - 1);
      const uint32_t off = (uint32_t)list[j] * kTealBlock;  // d_in * 128 < 2^32
      w0[u].load(W0 + off);
      if constexpr (DUAL) w1[u].load(W1 + off);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * kTbGroups + g;
      const float h = j < m ? xl[min(j, m - 1)] : 0.f;
      float f[8];
      w0[u].to_float(f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc0[e] = fmaf(h, f[e], acc0[e]);
      if constexpr (DUAL) {
        w1[DUAL ? u : 0].to_float(f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc1[e] = fmaf(h, f[e], acc1[e]);
      }
    }
  }

  // 3. the row groups in a fixed order, then this slice's partial sums
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[g][8 * q + e] = acc0[e];
    if constexpr (DUAL) red[g][kTealBlock + 8 * q + e] = acc1[e];
  }
  __syncthreads();
  const int bw = nblk * kTealBlock;                  // a slice's partial width per matrix
  float* part = a.part + (size_t)s * bw;
  if (threadIdx.x < NCOL) {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < kTbGroups; ++k) v += red[k][threadIdx.x];
    const int mat = threadIdx.x / kTealBlock, cc = threadIdx.x % kTealBlock;
    store_agent(part + (size_t)mat * S * bw + b * kTealBlock + cc, v);
    __builtin_amdgcn_s_waitcnt(0);  // stored before the ticket
  }
  __syncthreads();
  if (threadIdx.x == 0)
    tk_s = __hip_atomic_fetch_add(a.tickets + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (tk_s != (unsigned)(S - 1)) return;  // workgroup-uniform: not the block's last slice

  // 4. the block's column sums over the slices, in slice order
  if (threadIdx.x < NCOL) {
    const int mat = threadIdx.x / kTealBlock, cc = threadIdx.x % kTealBlock;
    const float* p = a.part + (size_t)mat * S * bw + b * kTealBlock + cc;
    col[threadIdx.x] = sum_agent(p, bw, S);
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(a.tickets + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int cb = b * kTealBlock;
  if constexpr (EPI == TEAL_STORE || ACC) {
    if (threadIdx.x < NCOL) {
      const int mat = threadIdx.x / kTealBlock, c = cb + threadIdx.x % kTealBlock;
      float* y = mat ? a.y2 : a.y;
      if (c < d_out) y[c] = y_old + col[threadIdx.x];
    }
  } else if constexpr (EPI == TEAL_SWIGLU) {
    if (threadIdx.x < kTealBlock) {
      const int c = cb + threadIdx.x;
      if (c < d_out) {
        const float h = silu(col[threadIdx.x]) * col[kTealBlock + threadIdx.x];
        a.y[c] = h;
        if (a.keep_next) a.keep_next[c] = a.t_next < 0.f || fabsf(h) > a.t_next;
      }
    }
  } else {  // TEAL_QKV: rotation pairs (i, i + d_h/2) of the heads within the block
    const QkvArgs& qa = a.qkv;
    const int dh = qa.dh, half = dh >> 1;
    if (threadIdx.x < kTealBlock / 2) {
      const int hb = threadIdx.x / half;            // head within the block
      const int i = threadIdx.x - hb * half;
      const int head = (cb / dh) + hb;
      const int ca = hb * dh + i;                   // block-local columns of the pair
      if (cb + ca < d_out) {
        float va = col[ca], vb = col[ca + half];
        if (head < qa.h_q + qa.h_kv) {  // rotate q and k, not v
          const float cs = qa.rope.c[i], sn = qa.rope.s[i];
          const float ra = va * cs - vb * sn, rb = vb * cs + va * sn;
          va = ra;
          vb = rb;
        }
        if (head < qa.h_q) {
          qa.q_out[head * dh + i] = va;
          qa.q_out[head * dh + i + half] = vb;
        } else {
          const bool is_k = head < qa.h_q + qa.h_kv;
          const int kv = is_k ? head - qa.h_q : head - qa.h_q - qa.h_kv;
          KT* full = static_cast<KT*>(is_k ? qa.k_full : qa.v_full);
          const size_t off = ((size_t)kv * qa.cap_full + qa.row_full) * dh + i;
          store_elem(full + off, va);
          store_elem(full + off + half, vb);
          if (qa.k_sel) {
            KT* sel = static_cast<KT*>(is_k ? qa.k_sel : qa.v_sel);
            // ragged budgets: each KV head appends at its own row
            const int rsel = qa.ragged ? qa.sel_rows.v[kv & (kMaxKvHeads - 1)] : qa.row_sel;
            const size_t offs = ((size_t)kv * qa.cap_sel + rsel) * dh + i;
            store_elem(sel + offs, va);
            store_elem(sel + offs + half, vb);
          }
        }
      }
    }
  }
}

__global__ void teal_zero_kernel(unsigned* __restrict__ t, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) t[i] = 0u;
}

// Slices per projection: the most that keep every compute unit at one
// workgroup at most (S * nblk <= CUs), within kTealMaxRange and at least 8
// channels per slice and kTealMaxSlices slices.  A 512-thread workgroup
// streams with eight waves; a second workgroup on a unit adds its own
// partial sums, ticket and staging more than it adds bandwidth.  Measured
// at 8B-class widths, 50% kept, in the step at 131072 context: QKV 5
// slices 10.4-10.6 us, against 11.5 for 4, 11.3-11.9 for 8, 11.6 for 10;
// O 8 slices 8.5-9.5 us against 10.1 for 12 and 11.7 for 16; gate + up 2
// slices 24.6 us against 27.3 for 3 and 25.6-25.9 for 4; the down
// projection 8 slices (composed step 2507-2522 us) against 7 (2542-2544),
// 10 (2569) and 16 (2541-2548).
int teal_slices(int d_in, int d_out) {
  const int nblk = (d_out + kTealBlock - 1) / kTealBlock;
  const int lo = (d_in + kTealMaxRange - 1) / kTealMaxRange;
  int hi = d_in / 8;
  if (hi > kTealMaxSlices) hi = kTealMaxSlices;
  if (hi < lo) hi = lo;
  int s = cu_count_dev() / nblk;
  if (s < lo) s = lo;
  if (s > hi) s = hi;
  return s < 1 ? 1 : s;
}

template <typename WT, bool DUAL, typename KT>
static void teal_typed(const TealArgs& a, hipStream_t s) {
  const dim3 grid(teal_slices(a.d_in, a.d_out), (a.d_out + kTealBlock - 1) / kTealBlock);
  switch (a.epi) {
    case TEAL_STORE:
      launch_kernel(a.kind, teal_kernel<WT, DUAL, TEAL_STORE, KT>, grid, dim3(kTbThreads), 0, s, a);
      break;
    case TEAL_ACC:
      launch_kernel(a.kind, teal_kernel<WT, DUAL, TEAL_ACC, KT>, grid, dim3(kTbThreads), 0, s, a);
      break;
    case TEAL_DOWN:
      if constexpr (!DUAL)
        launch_kernel(a.kind, teal_kernel<WT, false, TEAL_DOWN, KT>, grid,
                      dim3(kTbThreads), 0, s, a);
      break;
    case TEAL_CATS_DOWN:
      if constexpr (!DUAL)
        launch_kernel(a.kind, teal_kernel<WT, false, TEAL_CATS_DOWN, KT>, grid,
                      dim3(kTbThreads), 0, s, a);
      break;
    case TEAL_SWIGLU:
      if constexpr (DUAL)
        launch_kernel(a.kind, teal_kernel<WT, true, TEAL_SWIGLU, KT>, grid, dim3(kTbThreads), 0,
                      s, a);
      break;
    default:
      if constexpr (!DUAL)
        launch_kernel(a.kind, teal_kernel<WT, false, TEAL_QKV, KT>, grid, dim3(kTbThreads), 0, s,
                      a);
      break;
  }
}

void launch_teal(const TealArgs& a, int w_dtype, int kv_dtype, hipStream_t s) {
  const bool dual = a.w1 != nullptr;
  if (a.epi == TEAL_QKV) {  // single matrix; the cache type matters
    if (w_dtype == 1) {
      if (kv_dtype == 1) teal_typed<bf16_t, false, bf16_t>(a, s);
      else teal_typed<bf16_t, false, float>(a, s);
    } else {
      if (kv_dtype == 1) teal_typed<float, false, bf16_t>(a, s);
      else teal_typed<float, false, float>(a, s);
    }
    return;
  }
  if (w_dtype == 1) {
    if (dual) teal_typed<bf16_t, true, float>(a, s);
    else teal_typed<bf16_t, false, float>(a, s);
  } else {
    if (dual) teal_typed<float, true, float>(a, s);
    else teal_typed<float, false, float>(a, s);
  }
}

void launch_teal_zero(unsigned* tickets, int n, hipStream_t s) {
  launch_kernel(K_TEAL_ZERO, teal_zero_kernel, dim3(1), dim3(256), 0, s, tickets, n);
}

}  // namespace sd
