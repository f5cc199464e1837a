// Batched projections on the matrix cores (gfx950, wave64).
//
// "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM Decoding",
// §3.3 "Dispatch and batching" and §4.4 "Batching": B sequences share every
// weight read.  At B = 8 each weight element feeds eight products.  On the
// vector ALUs (unpacked float32) that is as much arithmetic as the SIMDs issue
// while HBM streams the weights, so here the batched projections run as one
// matrix product Y [rows, B] = W [rows, d_in] X [d_in, B] on
// v_mfma_f32_16x16x32_bf16, and the vector ALUs only stage the inputs.
//
// Weight layout ("tiles").  W is cut into tiles of 16 rows and steps of 32
// input channels.  The 1 KB of one (tile, step) is stored in the A-operand
// order of the matrix core (lane l: row l % 16, channels 8 (l / 16) .. + 7 of
// the step), step-major: element (r, c) at
//   ((c / 32) T + r / 16) 512 + ((r % 16) + 16 ((c % 32) / 8)) 8 + c % 8
// with T = ceil(rows / 16) and padding rows and channels zero.  One wave load
// instruction reads 1 KB of contiguous memory straight into operand
// registers, and at each step a workgroup's eight waves read eight adjacent
// KB.  (Tile-major order, each tile's steps contiguous, put the eight streams
// of a workgroup 128 KB apart; measured with no other work, 8-wave
// workgroups then streamed at 4.8-5.1 TB/s against 6.8-6.9 TB/s step-major,
// at every grid size.)
//
// Inputs.  A float32 input x_b (times the RMSNorm weights) is split into three
// bf16 parts, hi + mid + lo == x_b exactly.  Column p NB + b of the B operand
// holds part p of sequence b, so one product yields all three; every product
// of two bf16 values is exact in float32, and the result hi + (mid + lo) has
// float32 accuracy.  The RMSNorm scale of sequence b is one number per
// sequence, applied to the finished sums.
//
// bmma_kernel: grid (KS input slices, row groups of 8 tiles), eight waves;
// wave w owns tile 8 g + w of row group g.
//   1. the wave streams its tile's fragments of the slice (8, 16 or 32
//      steps, T KB apart) in chunks of four 1 KB loads, four chunks in
//      flight: chunk c + 4 is issued as soon as chunk c has gone into the
//      products;
//   2. before the products, wave b stages sequence b's inputs of the slice as
//      B fragments in LDS (load, norm weights, split; the input loads are
//      issued before the first weight chunk) and adds up its x^2 for the
//      RMSNorm;
//   3. per step, NM = ceil(3 NB / 16) products per matrix;
//   4. the three parts of each sum are added; the slice's partial sums (and
//      x^2 sums) are stored at agent scope, then the workgroup takes its row
//      group's ticket;
//   5. the slice that draws the group's last ticket adds the KS partials in
//      slice order and applies the epilogue: y = (QKV), or for QKV with
//      128-dim heads (a row group is one head) RoPE at each sequence's
//      position with q written out and k, v appended to its caches; y += (O
//      and down, the residual); or the CATS gate: a = SiLU(gate), keep_b =
//      |a_b| > t, hmid_b = keep_b ? a_b up_b : 0, and the union of the keeps.
// The slice length (8, 16 or 32 steps) is chosen per launch so that the grid
// covers every compute unit and the chip holds it at once: every workgroup
// streams from the start and none waits for a second round.  Gate + up takes
// 64-step slices instead when that grid keeps every unit at one workgroup.
// No workgroup waits for another, and the summation order is fixed.
// Gate, up and down are read whole: at the batch sizes that need this path
// the union of the masks keeps nearly every channel, and the channels it
// drops are too few and too scattered to skip 16 rows or 32 channels at a
// time.
#include <math.h>

#include <map>
#include <mutex>

#include "common.hpp"
#include "internal.hpp"

namespace sd {

constexpr int kMmRows = 16;                        // rows per tile
constexpr int kMmK = 32;                           // input channels per step
constexpr int kMmWaves = 8;                        // tiles per row group
constexpr int kMmThreads = kMmWaves * kWave;       // 512
constexpr int kMmGroupRows = kMmWaves * kMmRows;   // 128
constexpr int kMmHeadDim = kMmGroupRows;           // the fused QKV and O paths' head size
constexpr int kMmNB = 8;                           // partial-sum stride in sequences
constexpr int kMmChunk = 4;                        // fragment loads per wave and chunk (4 KB)
constexpr int kMmDepth = 4;                        // chunks in flight per wave
constexpr int kMmMinSlice = 8;                     // steps per slice: 8, 16 or 32

int bmma_groups(int rows) {
  const int ntiles = (rows + kMmRows - 1) / kMmRows;
  return (ntiles + kMmWaves - 1) / kMmWaves;
}

// Slices for a slice length of ch steps.
static int mm_slices(int d_in, int ch) {
  const int nsteps = (d_in + kMmK - 1) / kMmK;
  return (nsteps + ch - 1) / ch;
}

// Buffers are sized for the shortest slices (the most partial sums).
size_t bmma_part_floats(int rows, int d_in, bool dual) {
  const size_t rows_pad = (size_t)((rows + kMmRows - 1) / kMmRows) * kMmRows;
  return (size_t)(dual ? 2 : 1) * mm_slices(d_in, kMmMinSlice) * kMmNB * rows_pad;
}

size_t bmma_ssq_floats(int rows, int d_in, bool dual) {
  (void)dual;
  return (size_t)bmma_groups(rows) * mm_slices(d_in, kMmMinSlice) * kMmNB;
}

// Sum of the three parts of sequence b = lane % 16 (lanes with lane % 16 >= NB
// hold nothing useful): hi in column b, mid in column NB + b, lo in column
// 2 NB + b (of the second product when NB = 8).
template <int NB, int NM>
__device__ __forceinline__ void mm_parts(const f32x4 (&c)[NM], float (&y)[4]) {
  static_assert(NB == 2 || NB == 4 || NB == 8, "batch templates 2, 4, 8");
  const int lane = lane_id(), base = lane & ~15, n = lane & 15;
  const int src_mid = base + ((n + NB) & 15);
  const int src_lo = base + ((n + 2 * NB) & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float hi = c[0][i];
    const float mid = __shfl(c[0][i], src_mid);
    float lo;
    if constexpr (2 * NB >= 16) lo = c[NM - 1][i];
    else lo = __shfl(c[0][i], src_lo);
    y[i] = hi + (mid + lo);
  }
}

// Fragment loads of chunk c of a wave's slice: four steps of one matrix, or
// two steps of each of two (gate and up); steps past the last repeat it
// (their inputs are zero).  Step j of the wave's tile is T KB after step j - 1.
template <bool DUAL>
__device__ __forceinline__ void mm_load_chunk(const u32x4* W0, const u32x4* W1, int j0, int c,
                                              int nsteps, int ntiles, u32x4 (&A)[kMmChunk]) {
  constexpr int SC = DUAL ? kMmChunk / 2 : kMmChunk;  // steps per chunk
#pragma unroll
  for (int f = 0; f < kMmChunk; ++f) {
    const int step = c * SC + (DUAL ? f / 2 : f);
    const size_t off = (size_t)min(j0 + step, nsteps - 1) * ntiles * kWave;
    A[f] = __builtin_nontemporal_load(((DUAL && (f & 1)) ? W1 : W0) + off);
  }
}

template <int NB, bool DUAL, int EPI, int CH>
__global__ __launch_bounds__(kMmThreads) void bmma_kernel(BmmaArgs a) {
  constexpr int SC = DUAL ? kMmChunk / 2 : kMmChunk;  // steps per chunk
  constexpr int NCH = CH / SC;                        // chunks per slice
  constexpr int NM = (3 * NB + 15) / 16;              // products per step and matrix
  constexpr int NMAT = DUAL ? 2 : 1;
  __shared__ u32x4 bfr[NM][CH][kWave];
  __shared__ float ys[NMAT][NB][kMmGroupRows];
  __shared__ float rs_s[NB];
  __shared__ unsigned tk_s;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int KS = gridDim.x, s = blockIdx.x, g = blockIdx.y;
  const int d_in = a.d_in, rows = a.rows, nb = a.nb;
  const int nsteps = (d_in + kMmK - 1) / kMmK;
  const int ntiles = (rows + kMmRows - 1) / kMmRows;
  const int rows_pad = ntiles * kMmRows;
  const int t_raw = g * kMmWaves + wave;
  const int tile = min(t_raw, ntiles - 1);
  const int j0 = s * CH;
  const u32x4* W0 = static_cast<const u32x4*>(a.w0) + (size_t)tile * kWave + lane;
  const u32x4* W1 = DUAL ? static_cast<const u32x4*>(a.w1) + (size_t)tile * kWave + lane : W0;

  // 1. the inputs first, then the first chunks of weights: a wave's loads
  //    return in issue order, so the staging below waits for the inputs only
  //    (behind a weight chunk it waited, at launch, for the whole chip's
  //    first burst of weight loads)
  u32x4 A[kMmDepth][kMmChunk];

  // 2. B fragments: wave b stages sequence b, lane l the slice's 8-channel
  //    groups l, l + 64, ...; column p NB + b holds part p
  constexpr int G = CH * 4 > kWave ? CH * 4 / kWave : 1;  // groups per lane
  float xv[G][8], nv[G][8];
  bool ok[G];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int e8 = lane + kWave * gi, k = j0 * kMmK + 8 * e8;
    ok[gi] = wave < nb && e8 < CH * 4 && k < d_in;  // d_in % 8 == 0: the group is whole
#pragma unroll
    for (int e = 0; e < 8; ++e) xv[gi][e] = nv[gi][e] = 0.f;
    if constexpr (EPI == MM_OMERGE) {
      // the merged attention output of head k / 128, columns k % 128 .. + 7:
      // the sequence's split partials combined with the weights
      // 2^(m_sp - max m) as the split-K combine does, online over the splits
      if (ok[gi]) {
        const int col = k % kMmHeadDim;
        const size_t hb = ((size_t)wave * a.h_q + k / kMmHeadDim) * a.m_stride;
        const int ns = a.m_splits[wave];
        float M = -INFINITY, L = 0.f, acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        for (int sp0 = 0; sp0 < ns; sp0 += 4) {
          float mv[4], lv[4], vv[4][8];
#pragma unroll
          for (int u = 0; u < 4; ++u) {  // the loads of four splits first
            const size_t sp = hb + min(sp0 + u, ns - 1);
            mv[u] = a.pm[sp];
            lv[u] = a.pl[sp];
            load8f(a.pacc + sp * kMmHeadDim + col, vv[u]);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (sp0 + u >= ns || mv[u] == -INFINITY) continue;  // past the end, or empty
            const float mn = fmaxf(M, mv[u]);
            const float so = M == -INFINITY ? 0.f : exp2f(M - mn), w = exp2f(mv[u] - mn);
            L = fmaf(L, so, w * lv[u]);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = fmaf(acc[e], so, w * vv[u][e]);
            M = mn;
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[gi][e] = acc[e] / L;
      }
    } else if (ok[gi]) {
      load8f(a.x + (size_t)wave * d_in + k, xv[gi]);
      if (a.norm) load8f(a.norm + k, nv[gi]);
    }
  }
#pragma unroll
  for (int c = 0; c < kMmDepth; ++c)
    if (c < NCH) mm_load_chunk<DUAL>(W0, W1, j0, c, nsteps, ntiles, A[c]);
  float ss = 0.f;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int e8 = lane + kWave * gi;
    if (wave < NB && e8 < CH * 4) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss = fmaf(xv[gi][e], xv[gi][e], ss);
        v[e] = a.norm ? xv[gi][e] * nv[gi][e] : xv[gi][e];
      }
      u32x4 part[3];
      split3_bf16(v, part[0], part[1], part[2]);
      const int jj = e8 >> 2, q = e8 & 3;
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const int c = p * NB + wave;
        bfr[c / 16][jj][(c % 16) + 16 * q] = part[p];
      }
    }
  }
  {
    constexpr int NZ = 16 * NM - 3 * NB;  // columns past the parts: zero
    for (int u = threadIdx.x; u < NZ * CH * 4; u += kMmThreads) {
      const int c = 3 * NB + u / (CH * 4), r = u % (CH * 4);
      bfr[c / 16][r >> 2][(c % 16) + 16 * (r & 3)] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  if (a.norm) ss = wave_sum(ss);
  __syncthreads();

  // 3. the products, chunk by chunk; chunk c + 4 is loaded into the registers
  //    chunk c has just been used from
  f32x4 c0[NM], c1[DUAL ? NM : 1];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    c0[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (DUAL) c1[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
#pragma unroll
    for (int u = 0; u < SC; ++u) {
      const int j = c * SC + u;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const u32x4 bv = bfr[m][j][lane];
        if constexpr (DUAL) {
          c0[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(A[c % kMmDepth][2 * u]),
                                                          as_bf16x8(bv), c0[m], 0, 0, 0);
          c1[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(A[c % kMmDepth][2 * u + 1]),
                                                          as_bf16x8(bv), c1[m], 0, 0, 0);
        } else {
          c0[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(A[c % kMmDepth][u]), as_bf16x8(bv),
                                                          c0[m], 0, 0, 0);
        }
      }
    }
    if (c + kMmDepth < NCH)
      mm_load_chunk<DUAL>(W0, W1, j0, c + kMmDepth, nsteps, ntiles, A[c % kMmDepth]);
  }

  // 4. the parts added, staged in LDS per row group, then this slice's
  //    partials part[mat][s][b][row] stored with consecutive threads on
  //    consecutive rows (whole lines per store instruction: every agent-scope
  //    store is written through on its own)
  float y0[4], y1[4];
  mm_parts<NB, NM>(c0, y0);
  if constexpr (DUAL) mm_parts<NB, NM>(c1, y1);
  const int n = lane & 15, q = lane >> 4;
  if (n < NB) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ys[0][n][wave * kMmRows + 4 * q + i] = y0[i];
      if constexpr (DUAL) ys[1][n][wave * kMmRows + 4 * q + i] = y1[i];
    }
  }
  __syncthreads();
  const size_t mat_stride = (size_t)KS * kMmNB * rows_pad;
  for (int u = threadIdx.x; u < NMAT * NB * kMmGroupRows; u += kMmThreads) {
    const int r = u % kMmGroupRows, b = (u / kMmGroupRows) % NB, mat = u / (kMmGroupRows * NB);
    const int row = g * kMmGroupRows + r;  // rows of clamped tiles lie past rows_pad
    if (b < nb && row < rows_pad)
      store_agent(a.part + mat * mat_stride + ((size_t)s * kMmNB + b) * rows_pad + row,
                  ys[mat][b][r]);
  }
  if (a.norm && wave < NB && lane == 0)
    store_agent(a.ssq + ((size_t)g * KS + s) * kMmNB + wave, ss);
  __builtin_amdgcn_s_waitcnt(0);  // stored before the ticket
  __syncthreads();
  if (threadIdx.x == 0)
    tk_s = __hip_atomic_fetch_add(a.tickets + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (tk_s != (unsigned)(KS - 1)) return;  // workgroup-uniform: not the group's last slice

  // 5. the group's sums over the slices, in slice order.  The compiler keeps
  //    agent-scope loads in order and waits for each before its first use, so
  //    every load of a batch (the thread's sums over up to 16 slices, and
  //    the x^2 sums) is issued before the first add: one round trip per batch
  //    instead of one per sum
  constexpr int NU = NMAT * NB * kMmGroupRows;            // sums of the group
  constexpr int IPT = (NU + kMmThreads - 1) / kMmThreads;  // sums per thread
  constexpr int KB = 32 / IPT < 16 ? 32 / IPT : 16;        // slices per batch
  const size_t sl_stride = (size_t)kMmNB * rows_pad;
  const bool has_ss = a.norm && threadIdx.x < NB;
  float acc[IPT], old[IPT], tot = 0.f;
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    acc[i] = 0.f;
    // the residual the sums are added to, loaded with the first batch (a
    // single matrix: the thread's sums are the outputs it writes)
    const int u = threadIdx.x + i * kMmThreads, b = u / kMmGroupRows;
    const int row = g * kMmGroupRows + u % kMmGroupRows;
    old[i] = (EPI == MM_RESID || EPI == MM_OMERGE) && u < NU && b < nb && row < rows
                 ? a.out[(size_t)b * rows + row]
                 : 0.f;
  }
  for (int k0 = 0; k0 < KS; k0 += KB) {
    float t[IPT][KB], q[KB];
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      const int k = k0 + kk;
      q[kk] = has_ss && k < KS ? load_agent(a.ssq + ((size_t)g * KS + k) * kMmNB + threadIdx.x)
                               : 0.f;
#pragma unroll
      for (int i = 0; i < IPT; ++i) {
        const int u = threadIdx.x + i * kMmThreads;
        const int r = u % kMmGroupRows, b = (u / kMmGroupRows) % NB, mat = u / (kMmGroupRows * NB);
        const int row = g * kMmGroupRows + r;
        t[i][kk] = u < NU && b < nb && row < rows_pad && k < KS
                       ? load_agent(a.part + mat * mat_stride + (size_t)k * sl_stride +
                                    (size_t)b * rows_pad + row)
                       : 0.f;  // terms past KS add +0
      }
    }
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) tot += q[kk];
#pragma unroll
    for (int i = 0; i < IPT; ++i)
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) acc[i] += t[i][kk];
  }
  if (threadIdx.x < NB) rs_s[threadIdx.x] = a.norm ? 1.0f / sqrtf(tot / (float)d_in + a.eps) : 1.f;
  if constexpr (EPI == MM_SWIGLU || EPI == MM_QKV) {
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int u = threadIdx.x + i * kMmThreads;
      if (u < NU)
        ys[u / (kMmGroupRows * NB)][(u / kMmGroupRows) % NB][u % kMmGroupRows] = acc[i];
    }
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(a.tickets + g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if constexpr (EPI == MM_STORE || EPI == MM_RESID || EPI == MM_OMERGE) {
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int u = threadIdx.x + i * kMmThreads, b = u / kMmGroupRows;
      const int row = g * kMmGroupRows + u % kMmGroupRows;
      if (u < NU && b < nb && row < rows) {
        const float v = rs_s[b] * acc[i];
        a.out[(size_t)b * rows + row] = EPI == MM_STORE ? v : old[i] + v;
      }
    }
  } else if constexpr (EPI == MM_QKV) {
    // row group g is head g: thread (b, i) rotates pair (i, i + 64) of
    // sequence b, then writes q or appends k, v (bf16) to b's caches
    constexpr int DH = kMmHeadDim, HALF = DH / 2;
    const int b = threadIdx.x / HALF, i = threadIdx.x % HALF, head = g;
    if (b < nb) {
      float lo = rs_s[b] * ys[0][b][i], hi = rs_s[b] * ys[0][b][i + HALF];
      if (head < a.h_q + a.h_kv && a.theta > 0.f) {
        const float2 r = a.rope_cs[b * HALF + i];
        const float c = r.x, sn = r.y;
        const float l2 = lo * c - hi * sn, h2 = hi * c + lo * sn;
        lo = l2;
        hi = h2;
      }
      if (head < a.h_q) {
        float* dst = a.q_out + ((size_t)b * a.h_q + head) * DH;
        dst[i] = lo;
        dst[i + HALF] = hi;
      } else {
        const bool is_k = head < a.h_q + a.h_kv;
        const int kv = is_k ? head - a.h_q : head - a.h_q - a.h_kv;
        bf16_t* full = static_cast<bf16_t*>(is_k ? a.kvs.k_full[b] : a.kvs.v_full[b]);
        bf16_t* row = full + ((size_t)kv * a.kvs.cap_full[b] + a.kvs.row_full[b]) * DH;
        store_elem(row + i, lo);
        store_elem(row + i + HALF, hi);
        bf16_t* sel = static_cast<bf16_t*>(is_k ? a.kvs.k_sel[b] : a.kvs.v_sel[b]);
        if (sel) {
          bf16_t* srow = sel + ((size_t)kv * a.kvs.cap_sel[b] + a.kvs.row_sel[b]) * DH;
          store_elem(srow + i, lo);
          store_elem(srow + i + HALF, hi);
        }
      }
    }
  } else {  // MM_SWIGLU: the CATS gate per sequence, the union per row
    for (int r = threadIdx.x; r < kMmGroupRows; r += kMmThreads) {
      const int row = g * kMmGroupRows + r;
      if (row >= rows) continue;
      uint32_t un = 0u;
      for (int b = 0; b < nb; ++b) {
        const float act = silu(rs_s[b] * ys[0][b][r]);
        const bool kb = a.t < 0.f || fabsf(act) > a.t;
        const size_t o = (size_t)b * rows + row;
        a.act[o] = act;
        a.keep[o] = kb ? 1 : 0;
        a.hmid[o] = kb ? act * (rs_s[b] * ys[DUAL ? 1 : 0][b][r]) : 0.f;
        un |= kb ? 1u : 0u;
      }
      a.uni[row] = (uint8_t)un;
    }
  }
}

// W [rows, d_in] bf16 row-major -> tiles (step-major); one thread per 16-byte
// fragment.
__global__ void pack_tiles_kernel(const bf16_t* __restrict__ w, int rows, int d_in,
                                  u32x4* __restrict__ out, size_t n_frag) {
  const int ntiles = (rows + kMmRows - 1) / kMmRows;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_frag;
       i += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(i % kWave);
    const size_t ts = i / kWave;
    const int tile = (int)(ts % ntiles), step = (int)(ts / ntiles);
    const int r = tile * kMmRows + lane % 16, c = step * kMmK + 8 * (lane / 16);
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (r < rows && c < d_in) v = *reinterpret_cast<const u32x4*>(w + (size_t)r * d_in + c);
    out[i] = v;
  }
}

// Workgroups the chip holds at once for a kernel (occupancy query, cached).
template <typename K>
static int mm_resident(K kern) {
  static std::map<const void*, int> cache;
  static std::mutex mu;
  std::lock_guard<std::mutex> g(mu);
  auto it = cache.find((const void*)kern);
  if (it != cache.end()) return it->second;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kMmThreads, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const int slots = per_cu * cu_count_dev();
  cache[(const void*)kern] = slots;
  return slots;
}

// Slice length: the longest of 32, 16, 8 steps whose grid has a workgroup for
// every compute unit and fits on the chip at once (longer slices: fewer
// partial sums and a shorter final reduction; measured: 8-step slices on the
// narrow projections cost more in per-workgroup latency than they gained).
// If none does, 8 steps when even that grid leaves units idle, else 32.
template <int NB, bool DUAL, int EPI, int CH>
static bool mm_try(const BmmaArgs& a, hipStream_t s, int mode) {
  auto kern = bmma_kernel<NB, DUAL, EPI, CH>;
  const long long grid = (long long)bmma_groups(a.rows) * mm_slices(a.d_in, CH);
  if (mode == 0 && (grid < cu_count_dev() || grid > mm_resident(kern))) return false;
  launch_kernel(a.kind, kern, dim3(mm_slices(a.d_in, CH), bmma_groups(a.rows)),
                dim3(kMmThreads), 0, s, a);
  return true;
}

template <int NB, bool DUAL, int EPI>
static void mm_launch(const BmmaArgs& a, hipStream_t s) {
  // gate + up: 64-step slices when that keeps every compute unit at one
  // workgroup at most, each unit then streaming both matrices' rows with one
  // set of partial sums (measured at B = 8, 8B-class widths: 42.1-43.4 us
  // against 45.7-46.4 for 32-step slices, two workgroups on most units; the
  // same rule for down, 25.1-25.8 against 25.0, and QKV, 14.9 against 15.0,
  // gained nothing)
  if (DUAL && (long long)bmma_groups(a.rows) * mm_slices(a.d_in, 64) <= cu_count_dev() &&
      mm_try<NB, DUAL, EPI, 64>(a, s, 1))
    return;
  if (mm_try<NB, DUAL, EPI, 32>(a, s, 0)) return;
  if (mm_try<NB, DUAL, EPI, 16>(a, s, 0)) return;
  if (mm_try<NB, DUAL, EPI, 8>(a, s, 0)) return;
  if ((long long)bmma_groups(a.rows) * mm_slices(a.d_in, 8) < cu_count_dev())
    mm_try<NB, DUAL, EPI, 8>(a, s, 1);
  else
    mm_try<NB, DUAL, EPI, 32>(a, s, 1);
}

template <int NB>
static void bmma_nb(const BmmaArgs& a, hipStream_t s) {
  if (a.w1) mm_launch<NB, true, MM_SWIGLU>(a, s);
  else if (a.epi == MM_RESID) mm_launch<NB, false, MM_RESID>(a, s);
  else if (a.epi == MM_QKV) mm_launch<NB, false, MM_QKV>(a, s);
  else if (a.epi == MM_OMERGE) mm_launch<NB, false, MM_OMERGE>(a, s);
  else mm_launch<NB, false, MM_STORE>(a, s);
}

void launch_bmma(const BmmaArgs& a, hipStream_t s) {
  if (a.nb <= 2) bmma_nb<2>(a, s);
  else if (a.nb <= 4) bmma_nb<4>(a, s);
  else bmma_nb<8>(a, s);
}

void launch_pack_tiles(const void* w, int rows, int d_in, void* out, hipStream_t s) {
  const size_t n_frag = (size_t)((rows + kMmRows - 1) / kMmRows) *
                        ((d_in + kMmK - 1) / kMmK) * kWave;
  size_t blocks = (n_frag + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  launch_kernel(K_PACK_TILES, pack_tiles_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                static_cast<const bf16_t*>(w), rows, d_in, static_cast<u32x4*>(out), n_frag);
}

}  // namespace sd
