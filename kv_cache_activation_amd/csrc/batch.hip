// Batched decode: nb sequences (2..8) share every weight read (gfx950, wave64).
//
// "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding",
// §3.3 "Dispatch and batching" and §4.4 "Batching": a batch of B sequences
// reads each weight once for all of them, while every sequence reads its own
// cache; a sparse projection must then read every channel that at least one
// sequence keeps (the union of the masks).
//
// bgemv_kernel: y[b] = W x_b for all nb sequences, W row-major [rows, d_in].
//   A workgroup of eight waves stages the nb input vectors in LDS (times the
//   RMSNorm when given, zero-padded to a multiple of 512 columns), then each
//   wave takes two rows at a time: every lane loads 16 bytes per 512-column
//   chunk of both rows (all chunks issued together, no branch between them:
//   lanes past the row end read a clamped address against zero x), and
//   multiplies them with the nb vectors, so a weight byte read once feeds nb
//   dot products.  The grid is what the chip holds at once and the waves loop
//   over the rows, so the staging is paid once per workgroup.
//   Epilogues: store (the QKV outputs, for the RoPE kernel), residual add
//   (O: h_b += W_o attn_b), or the CATS gate: a = SiLU(W_gate x_b), keep_b =
//   |a| > t decided per sequence in float32, the union of the keeps, and for
//   every row some sequence keeps, the up rows read once for all sequences:
//   hmid_b = keep_b ? a_b (W_up x_b) : 0.
// brope_append_kernel: per (sequence, head) RoPE at the sequence's own
//   position (angles in double precision), q out, k and v rounded to the
//   cache type and appended to that sequence's full and gathered caches.
// The down projection over the union is down_kernel with nb sequences; split-K
// attention runs per sequence on that sequence's cache.
#include <math.h>

#include <map>
#include <mutex>

#include "common.hpp"
#include "internal.hpp"

namespace sd {

constexpr int kBThreads = 512;
constexpr int kBWaves = kBThreads / kWave;
constexpr int kBRows = 2;  // rows per wave at a time

enum { BM_STORE = 0, BM_RESID = 1, BM_GATE = 2 };

// Row dot products of kBRows weight rows with the NB staged vectors:
// acc[r][b] = W[row[r]] . xs[b] (every lane ends with the full sums).  The
// chunks go in groups of up to four: a group's loads (both rows) are issued
// together, then multiplied with the nb vectors.
template <typename WT, int NB, int NCH>
__device__ __forceinline__ void brow_dots(const WT* __restrict__ W, const int (&row)[kBRows],
                                          int d_in, const float* xs, float (&acc)[kBRows][NB]) {
  constexpr int XW = NCH * 512;
  constexpr int CG = NCH < 4 ? NCH : 4;
  const int lane = lane_id();
#pragma unroll
  for (int r = 0; r < kBRows; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
#pragma unroll
  for (int c0 = 0; c0 < NCH; c0 += CG) {
    // one group's loads at a time: hoisting the next group's loads above this
    // group's FMAs would need twice the registers (and spills with the gate)
    if (c0) asm volatile("" ::: "memory");
    Vec8<WT> g[kBRows][CG];
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      const int col = min((c0 + c) * 512 + 8 * lane, d_in - 8);
#pragma unroll
      for (int r = 0; r < kBRows; ++r) g[r][c].load(W + (size_t)row[r] * d_in + col);
    }
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      float f[kBRows][8];
#pragma unroll
      for (int r = 0; r < kBRows; ++r) g[r][c].to_float(f[r]);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float xv[8];
        load8f(xs + b * XW + (c0 + c) * 512 + 8 * lane, xv);
#pragma unroll
        for (int r = 0; r < kBRows; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r][b] = fmaf(f[r][e], xv[e], acc[r][b]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kBRows; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = wave_sum(acc[r][b]);
}

template <typename WT, int NB, int NCH, bool GATE>
__global__ __launch_bounds__(kBThreads) void bgemv_kernel(
    const float* __restrict__ X, int nb, int d_in, const float* __restrict__ nw, float eps,
    const WT* __restrict__ W, int rows, int mode, float* __restrict__ out,
    const WT* __restrict__ Wu, float t, float* __restrict__ act, uint8_t* __restrict__ keep,
    uint8_t* __restrict__ uni, float* __restrict__ hmid) {
  constexpr int XW = NCH * 512;
  extern __shared__ float xs[];  // [NB][XW]
  __shared__ float red[kBWaves][NB];
  const int lane = lane_id(), wave = threadIdx.x / kWave;

  // stage the inputs (float4 pieces; zero past d_in and for b >= nb)
  float ss[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) ss[b] = 0.f;
  for (int i4 = threadIdx.x; i4 < XW / 4; i4 += kBThreads) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (b < nb && 4 * i4 < d_in) v = reinterpret_cast<const float4*>(X + (size_t)b * d_in)[i4];
      reinterpret_cast<float4*>(xs + b * XW)[i4] = v;
      ss[b] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
  }
  if (nw) {  // RMSNorm per sequence: x * rsqrt(mean(x^2) + eps) * nw
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float sw = wave_sum(ss[b]);
      if (lane == 0) red[wave][b] = sw;
    }
    __syncthreads();
    float rs[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < kBWaves; ++w) tot += red[w][b];
      rs[b] = rsqrtf(tot / (float)d_in + eps);
    }
    for (int i4 = threadIdx.x; i4 < XW / 4; i4 += kBThreads) {
      float4 n = make_float4(0.f, 0.f, 0.f, 0.f);
      if (4 * i4 < d_in) n = reinterpret_cast<const float4*>(nw)[i4];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float4 v = reinterpret_cast<float4*>(xs + b * XW)[i4];
        v.x *= rs[b] * n.x; v.y *= rs[b] * n.y; v.z *= rs[b] * n.z; v.w *= rs[b] * n.w;
        reinterpret_cast<float4*>(xs + b * XW)[i4] = v;
      }
    }
  }
  __syncthreads();

  const int gw = blockIdx.x * kBWaves + wave, n_waves = gridDim.x * kBWaves;
  for (int r0 = gw * kBRows; r0 < rows; r0 += n_waves * kBRows) {
    // keeps the compiler from hoisting the staged x out of the loop into
    // registers (nb * d_in / 64 of them per lane): x is read from LDS per row
    asm volatile("" ::: "memory");
    int row[kBRows];
#pragma unroll
    for (int r = 0; r < kBRows; ++r) row[r] = min(r0 + r, rows - 1);
    float acc[kBRows][NB];
    brow_dots<WT, NB, NCH>(W, row, d_in, xs, acc);
    if constexpr (!GATE) {
      // lane r * NB + b writes (row r, sequence b)
#pragma unroll
      for (int r = 0; r < kBRows; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          if (lane == r * NB + b && b < nb && r0 + r < rows) {
            float* p = out + (size_t)b * rows + r0 + r;
            *p = mode == BM_RESID ? *p + acc[r][b] : acc[r][b];
          }
      continue;
    } else {
    // CATS gate: per-sequence activations and keeps, the union per row
    float a[kBRows][NB];
    bool any = false, kb[kBRows][NB];
    uint32_t un[kBRows];
#pragma unroll
    for (int r = 0; r < kBRows; ++r) {
      un[r] = 0u;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        a[r][b] = silu(acc[r][b]);
        kb[r][b] = b < nb && r0 + r < rows && (t < 0.f || fabsf(a[r][b]) > t);
        un[r] |= kb[r][b] ? 1u : 0u;
      }
      any = any || un[r];
    }
    float up[kBRows][NB];
    if (any) {  // wave-uniform: some sequence keeps one of the two rows
      brow_dots<WT, NB, NCH>(Wu, row, d_in, xs, up);
    } else {
#pragma unroll
      for (int r = 0; r < kBRows; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) up[r][b] = 0.f;
    }
#pragma unroll
    for (int r = 0; r < kBRows; ++r) {
      if (r0 + r >= rows) continue;
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (lane == r * NB + b && b < nb) {
          const size_t o = (size_t)b * rows + r0 + r;
          act[o] = a[r][b];
          keep[o] = kb[r][b] ? 1 : 0;
          hmid[o] = kb[r][b] ? a[r][b] * up[r][b] : 0.f;
        }
      if (lane == 0) uni[r0 + r] = (uint8_t)un[r];
    }
    }
  }
}

// One workgroup per (sequence, head): heads [0, h_q) are query heads, [h_q,
// h_q + h_kv) key heads, then value heads.  One thread per rotation pair.
template <typename KT>
__global__ void brope_append_kernel(const float* __restrict__ qkv, int qkv_out, int h_q, int h_kv,
                                    int dh, float theta, BatchKv kvs, float* __restrict__ q) {
  const int b = blockIdx.x, head = blockIdx.y, i = threadIdx.x, half = dh / 2;
  if (i >= half) return;
  const float* src = qkv + (size_t)b * qkv_out + (size_t)head * dh;
  float lo = src[i], hi = src[i + half];
  if (head < h_q + h_kv && theta > 0.f) {  // rotate-half pair (i, i + d_h / 2)
    float c, s;
    rope_cs(kvs.pos[b], i, dh, theta, c, s);
    const float l2 = lo * c - hi * s, h2 = hi * c + lo * s;
    lo = l2;
    hi = h2;
  }
  if (head < h_q) {
    float* dst = q + ((size_t)b * h_q + head) * dh;
    dst[i] = lo;
    dst[i + half] = hi;
    return;
  }
  const bool is_k = head < h_q + h_kv;
  const int kv = is_k ? head - h_q : head - h_q - h_kv;
  KT* full = (KT*)(is_k ? kvs.k_full[b] : kvs.v_full[b]);
  KT* row = full + ((size_t)kv * kvs.cap_full[b] + kvs.row_full[b]) * dh;
  store_elem(row + i, lo);
  store_elem(row + i + half, hi);
  KT* sel = (KT*)(is_k ? kvs.k_sel[b] : kvs.v_sel[b]);
  if (sel) {
    KT* srow = sel + ((size_t)kv * kvs.cap_sel[b] + kvs.row_sel[b]) * dh;
    store_elem(srow + i, lo);
    store_elem(srow + i + half, hi);
  }
}

// The rotations of every pair at each sequence's position, once per step.
__global__ void brope_table_kernel(BatchKv kvs, int dh, float theta, float2* __restrict__ cs) {
  const int b = blockIdx.x, i = threadIdx.x, half = dh / 2;
  if (i >= half) return;
  float c, s;
  rope_cs(kvs.pos[b], i, dh, theta, c, s);
  cs[b * half + i] = make_float2(c, s);
}

template <typename WT, int NB, int NCH, bool GATE>
static void bgemv_launch(const BgemvArgs& a, hipStream_t s) {
  auto kern = bgemv_kernel<WT, NB, NCH, GATE>;
  const uint32_t lds = (uint32_t)(NB * NCH * 512 * sizeof(float));
  static std::map<const void*, int> occ_cache;
  static std::mutex mu;
  int per_cu = 0;
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = occ_cache.find((const void*)kern);
    if (it == occ_cache.end()) {
      if (lds > 65536)
        (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kBThreads, lds) !=
              hipSuccess ||
          per_cu < 1)
        per_cu = 1;
      occ_cache[(const void*)kern] = per_cu;
    } else {
      per_cu = it->second;
    }
  }
  const int groups = (a.rows + kBWaves * kBRows - 1) / (kBWaves * kBRows);
  int grid = per_cu * cu_count_dev();
  if (grid > groups) grid = groups;
  launch_kernel(a.kind, kern, dim3(grid), dim3(kBThreads), lds, s, a.x, a.nb, a.d_in, a.norm,
                a.eps, (const WT*)a.w, a.rows, a.mode, a.out, (const WT*)a.w_up, a.t, a.act,
                a.keep, a.uni, a.hmid);
}

template <typename WT, int NB, bool GATE>
static void bgemv_nch(const BgemvArgs& a, hipStream_t s) {
  const int nch = (a.d_in + 511) / 512;
  if (nch <= 1) bgemv_launch<WT, NB, 1, GATE>(a, s);
  else if (nch <= 2) bgemv_launch<WT, NB, 2, GATE>(a, s);
  else if (nch <= 4) bgemv_launch<WT, NB, 4, GATE>(a, s);
  else bgemv_launch<WT, NB, 8, GATE>(a, s);
}

template <typename WT, int NB>
static void bgemv_nb(const BgemvArgs& a, hipStream_t s) {
  if (a.mode == BM_GATE) bgemv_nch<WT, NB, true>(a, s);
  else bgemv_nch<WT, NB, false>(a, s);
}

template <typename WT>
static void bgemv_typed(const BgemvArgs& a, hipStream_t s) {
  if (a.nb <= 2) bgemv_nb<WT, 2>(a, s);
  else if (a.nb <= 4) bgemv_nb<WT, 4>(a, s);
  else bgemv_nb<WT, 8>(a, s);
}

int cu_count_dev() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return cus > 0 ? cus : 256;
}

void launch_bgemv(const BgemvArgs& a, int w_dtype, hipStream_t s) {
  if (w_dtype == 1) bgemv_typed<bf16_t>(a, s);
  else bgemv_typed<float>(a, s);
}

void launch_brope_table(const BatchKv& kvs, int nb, int dh, float theta, float2* cs,
                        hipStream_t s) {
  launch_kernel(K_BATCH_ROPE, brope_table_kernel, dim3(nb), dim3(dh / 2), 0, s, kvs, dh, theta, cs);
}

void launch_brope_append(const float* qkv, int nb, int qkv_out, int h_q, int h_kv, int dh,
                         float theta, const BatchKv& kvs, float* q, int kv_dtype, hipStream_t s) {
  const dim3 grid(nb, h_q + 2 * h_kv), block(dh / 2);
  if (kv_dtype == 1)
    launch_kernel(K_BATCH_ROPE, brope_append_kernel<bf16_t>, grid, block, 0, s, qkv, qkv_out, h_q,
                  h_kv, dh, theta, kvs, q);
  else
    launch_kernel(K_BATCH_ROPE, brope_append_kernel<float>, grid, block, 0, s, qkv, qkv_out, h_q,
                  h_kv, dh, theta, kvs, q);
}

}  // namespace sd
