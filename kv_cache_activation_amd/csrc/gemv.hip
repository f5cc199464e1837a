// Weight-streaming GEMV kernels of the decode step (gfx950, wave64).
//
// Every kernel here reads one weight matrix once per step, the fixed term of
// the byte account in "Where Activation Sparsity and KV-Cache Sparsity Cross
// in LLM Decoding" (§1, §3.2).  Layout of the work:
//   * a workgroup stages its input vector in LDS once (x * norm weight) and
//     reduces sum(x^2) for the RMSNorm scale rs, applied to each dot product
//     at the end (RMSNorm(x) . w = rs * (x * norm) . w), so the norm costs no
//     extra pass over HBM;
//   * each wave keeps its slice of the input in VGPRs (lane l holds columns
//     8(l + 64k) .. +8) and streams weight rows with 16-byte loads, two rows in
//     flight per iteration, reducing each dot product across the wave;
//   * waves stride over rows, so any grid size covers any matrix.
#include "common.hpp"
#include "internal.hpp"

namespace sd {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

// Stage x (times the norm weights when `norm`) into LDS; return the RMSNorm
// scale 1/sqrt(mean(x^2) + eps), or 1 without norm.
__device__ float stage_input(const float* __restrict__ x, const float* __restrict__ nw, int d,
                             float eps, bool norm, float* xs) {
  __shared__ float red[kWavesPerBlock];
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    float v = x[i];
    ss += v * v;
    xs[i] = norm ? v * nw[i] : v;
  }
  ss = wave_sum(ss);
  if (lane_id() == 0) red[threadIdx.x / kWave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) tot += red[w];
  return norm ? 1.0f / sqrtf(tot / (float)d + eps) : 1.0f;
}

template <int NCH>
struct XSlice {
  float v[NCH][8];
  __device__ __forceinline__ void load(const float* xs, int d8) {
    const int lane = lane_id();
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      int c8 = lane + kWave * k;
      if (c8 < d8) {
        load8f(xs + 8 * c8, v[k]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[k][e] = 0.f;
      }
    }
  }
};

// R weight rows held by one wave: lane l holds the 16-byte chunks
// 8(l + 64k) .. +8 of each row, k < NCH.  load() only issues the loads, so the
// caller can overlap their latency with other work before dot().
// rows[r] < 0 marks an absent row (its dot product is 0).
template <typename WT, int NCH, int R>
struct RowBlock {
  Vec8<WT> w[R][NCH];

  __device__ __forceinline__ void load(const WT* __restrict__ W, int ld, const int (&rows)[R],
                                       int d8) {
    const int lane = lane_id();
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int k = 0; k < NCH; ++k) {
        const int c8 = lane + kWave * k;
        if (rows[r] >= 0 && c8 < d8) w[r][k].load(W + (size_t)rows[r] * ld + 8 * c8);
      }
  }

  __device__ __forceinline__ void dot(const XSlice<NCH>& x, int d8, const int (&rows)[R],
                                      float (&out)[R]) const {
    const int lane = lane_id();
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < NCH; ++k) {
        const int c8 = lane + kWave * k;
        if (rows[r] >= 0 && c8 < d8) {
          float f[8];
          w[r][k].to_float(f);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc = fmaf(f[e], x.v[k][e], acc);
        }
      }
      out[r] = wave_sum(acc);
    }
  }
};

// ------------------------------------------------------------------ QKV
// x = RMSNorm(h) * attn_norm; [q; k; v] = W_qkv x; RoPE on q and k at `pos`
// (rotate-half pairs (i, i + d_h/2), angles in double precision); q goes to
// q_out, k and v are rounded to the cache type and written at row row_full of
// the full cache and, when k_sel is given, at row row_sel of the gathered
// buffer.  A wave computes both rows of one rotation pair.  Block 0 also
// clears `zero_n` words of `zero_buf` for kernels later in the same step.
template <typename WT, typename KT, int NCH>
__global__ __launch_bounds__(kThreads) void qkv_rope_append_kernel(
    const float* __restrict__ h, const float* __restrict__ nw, float eps,
    const WT* __restrict__ W, int d, int h_q, int h_kv, int dh, float theta, int pos,
    float* __restrict__ q_out, KT* __restrict__ k_full, KT* __restrict__ v_full, int cap_full,
    int row_full, KT* __restrict__ k_sel, KT* __restrict__ v_sel, int cap_sel, int row_sel,
    unsigned* __restrict__ zero_buf, int zero_n) {
  extern __shared__ float xs[];
  __shared__ float rope_c[64], rope_s[64];
  const int half = dh >> 1;
  const int d8 = d >> 3;
  const int n_pairs = (h_q + 2 * h_kv) * half;
  const int wave = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  const int n_waves = gridDim.x * kWavesPerBlock;
  // issue this wave's first weight rows before the prologue: their latency
  // overlaps the norm reduction and the RoPE table
  RowBlock<WT, NCH, 2> blk;
  auto pair_rows = [&](int p, int (&rows)[2]) {
    const int head = p / half, i = p - head * half;
    rows[0] = p < n_pairs ? head * dh + i : -1;
    rows[1] = p < n_pairs ? head * dh + i + half : -1;
  };
  int rows[2];
  pair_rows(wave, rows);
  blk.load(W, d, rows, d8);

  if (blockIdx.x == 0 && zero_buf)
    for (int i = threadIdx.x; i < zero_n; i += blockDim.x) zero_buf[i] = 0u;
  // cos/sin of pos * theta^(-2i/d_h), in double precision: pos reaches 1e5+
  // and float angles would carry errors of order 1e-2 radians.
  if (threadIdx.x < half) {
    float c = 1.f, sn = 0.f;
    if (theta > 0.f) {
      const double inv_freq = pow((double)theta, -2.0 * (double)threadIdx.x / (double)dh);
      double sd, cd;
      sincos((double)pos * inv_freq, &sd, &cd);
      c = (float)cd;
      sn = (float)sd;
    }
    rope_c[threadIdx.x] = c;
    rope_s[threadIdx.x] = sn;
  }
  const float rs = stage_input(h, nw, d, eps, true, xs);
  __syncthreads();
  XSlice<NCH> x;
  x.load(xs, d8);

  for (int p = wave; p < n_pairs; p += n_waves) {
    const int head = p / half, i = p - head * half;
    if (p != wave) {
      pair_rows(p, rows);
      blk.load(W, d, rows, d8);
    }
    float s[2];
    blk.dot(x, d8, rows, s);
    if (lane_id() == 0) {
      float a = s[0] * rs, b = s[1] * rs;
      if (head < h_q + h_kv) {  // rotate q and k, not v
        const float c = rope_c[i], sn = rope_s[i];
        const float ra = a * c - b * sn;
        const float rb = b * c + a * sn;
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
        size_t off = ((size_t)kv * cap_full + row_full) * dh + i;
        store_elem(full + off, a);
        store_elem(full + off + half, b);
        if (k_sel) {
          KT* sel = is_k ? k_sel : v_sel;
          size_t offs = ((size_t)kv * cap_sel + row_sel) * dh + i;
          store_elem(sel + offs, a);
          store_elem(sel + offs + half, b);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ O
// h[r] += W_o[r] . attn  (residual add; attn is the attention output).
template <typename WT, int NCH>
__global__ __launch_bounds__(kThreads) void o_residual_kernel(const float* __restrict__ attn,
                                                              const WT* __restrict__ W, int din,
                                                              int dout, float* __restrict__ h) {
  extern __shared__ float xs[];
  const int d8 = din >> 3;
  const int wave = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  const int n_waves = gridDim.x * kWavesPerBlock;
  RowBlock<WT, NCH, 2> blk;
  int rows[2] = {2 * wave < dout ? 2 * wave : -1, 2 * wave + 1 < dout ? 2 * wave + 1 : -1};
  blk.load(W, din, rows, d8);  // before the prologue
  stage_input(attn, nullptr, din, 0.f, false, xs);
  __syncthreads();
  XSlice<NCH> x;
  x.load(xs, d8);
  for (int r0 = 2 * wave; r0 < dout; r0 += 2 * n_waves) {
    if (r0 != 2 * wave) {
      rows[0] = r0;
      rows[1] = r0 + 1 < dout ? r0 + 1 : -1;
      blk.load(W, din, rows, d8);
    }
    float s[2];
    blk.dot(x, d8, rows, s);
    if (lane_id() == 0) {
      h[r0] += s[0];
      if (rows[1] >= 0) h[r0 + 1] += s[1];
    }
  }
}

// ------------------------------------------------------------------ CATS gate + up
// x = RMSNorm(h) * mlp_norm (or x itself without norm); a_i = SiLU(W_gate[i] . x)
// (or a_i read from `act` when gate_in); channel i is kept iff t < 0 or
// |a_i| > t; for kept channels hmid_i = a_i (W_up[i] . x).  keep[i] is 1 or 0.
// With W_up == nullptr only `act` is produced (calibration).  `act` may
// be offset per block row for batched calibration (blockIdx.y states).
template <typename WT, int NCH>
__global__ __launch_bounds__(kThreads) void gate_up_kernel(
    const float* __restrict__ xin, const float* __restrict__ nw, float eps, int norm,
    const WT* __restrict__ Wg, const WT* __restrict__ Wu, int d, int dff, float t, int gate_in,
    int store_abs, float* __restrict__ act, uint8_t* __restrict__ keep, float* __restrict__ hmid,
    unsigned* __restrict__ zero_buf, int zero_n) {
  extern __shared__ float xs[];
  constexpr int R = 4;  // rows per wave iteration: their gate loads go out together
  xin += (size_t)blockIdx.y * d;
  act += (size_t)blockIdx.y * dff;
  const int d8 = d >> 3;
  const int lane = lane_id();
  const int wave = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  const int n_waves = gridDim.x * kWavesPerBlock;
  RowBlock<WT, NCH, R> blk;
  int rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = R * wave + r < dff ? R * wave + r : -1;
  if (!gate_in) blk.load(Wg, d, rows, d8);  // before the prologue

  if (blockIdx.x == 0 && blockIdx.y == 0 && zero_buf)
    for (int i = threadIdx.x; i < zero_n; i += blockDim.x) zero_buf[i] = 0u;
  const float rs = stage_input(xin, nw, d, eps, norm != 0, xs);
  __syncthreads();
  XSlice<NCH> x;
  x.load(xs, d8);
  for (int r0 = R * wave; r0 < dff; r0 += R * n_waves) {
    if (r0 != R * wave) {
#pragma unroll
      for (int r = 0; r < R; ++r) rows[r] = r0 + r < dff ? r0 + r : -1;
      if (!gate_in) blk.load(Wg, d, rows, d8);
    }
    float a[R];
    if (gate_in) {
#pragma unroll
      for (int r = 0; r < R; ++r) a[r] = rows[r] >= 0 ? act[rows[r]] : 0.f;
    } else {
      float g[R];
      blk.dot(x, d8, rows, g);
#pragma unroll
      for (int r = 0; r < R; ++r) a[r] = silu(g[r] * rs);
      if (lane == 0)
#pragma unroll
        for (int r = 0; r < R; ++r)
          if (rows[r] >= 0) act[rows[r]] = store_abs ? fabsf(a[r]) : a[r];
    }
    if (!Wu) continue;
    int urows[R];
    bool any = false;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool k = rows[r] >= 0 && (t < 0.f || fabsf(a[r]) > t);
      urows[r] = k ? rows[r] : -1;
      any |= k;
      if (lane == 0 && rows[r] >= 0) keep[rows[r]] = k;
    }
    if (!any) continue;
    blk.load(Wu, d, urows, d8);  // only the kept channels' up rows
    float u[R];
    blk.dot(x, d8, urows, u);
    if (lane == 0)
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (urows[r] >= 0) hmid[urows[r]] = a[r] * (u[r] * rs);
  }
}

// ------------------------------------------------------------------ launchers
static int nch_for(int d) {
  int need = (d / 8 + kWave - 1) / kWave;
  int n = 1;
  while (n < need) n <<= 1;
  return n;
}

#define SD_NCH_DISPATCH(D, ...)                 \
  switch (nch_for(D)) {                         \
    case 1: { constexpr int NCH = 1; __VA_ARGS__; } break;   \
    case 2: { constexpr int NCH = 2; __VA_ARGS__; } break;   \
    case 4: { constexpr int NCH = 4; __VA_ARGS__; } break;   \
    case 8: { constexpr int NCH = 8; __VA_ARGS__; } break;   \
    default: { constexpr int NCH = 16; __VA_ARGS__; } break; \
  }

template <typename WT, typename KT>
static void qkv_typed(const QkvArgs& a, hipStream_t s) {
  size_t lds = (size_t)a.d * sizeof(float);
  ProfScope prof(K_QKV, s);
  SD_NCH_DISPATCH(a.d, qkv_rope_append_kernel<WT, KT, NCH><<<a.grid, kThreads, lds, s>>>(
      a.h, a.norm, a.eps, (const WT*)a.w, a.d, a.h_q, a.h_kv, a.dh, a.theta, a.pos, a.q_out,
      (KT*)a.k_full, (KT*)a.v_full, a.cap_full, a.row_full, (KT*)a.k_sel, (KT*)a.v_sel,
      a.cap_sel, a.row_sel, a.zero_buf, a.zero_n));
}

void launch_qkv(const QkvArgs& a, int w_dtype, int kv_dtype, hipStream_t s) {
  if (w_dtype == 1 && kv_dtype == 1) qkv_typed<bf16_t, bf16_t>(a, s);
  else if (w_dtype == 1) qkv_typed<bf16_t, float>(a, s);
  else if (kv_dtype == 1) qkv_typed<float, bf16_t>(a, s);
  else qkv_typed<float, float>(a, s);
}

void launch_o(const float* attn, const void* w, int din, int dout, float* h, int w_dtype,
              int grid, hipStream_t s) {
  size_t lds = (size_t)din * sizeof(float);
  ProfScope prof(K_O, s);
  if (w_dtype == 1) {
    SD_NCH_DISPATCH(din, o_residual_kernel<bf16_t, NCH><<<grid, kThreads, lds, s>>>(
        attn, (const bf16_t*)w, din, dout, h));
  } else {
    SD_NCH_DISPATCH(din, o_residual_kernel<float, NCH><<<grid, kThreads, lds, s>>>(
        attn, (const float*)w, din, dout, h));
  }
}

void launch_gate_up(const GateUpArgs& a, int w_dtype, hipStream_t s) {
  size_t lds = (size_t)a.d * sizeof(float);
  dim3 grid(a.grid, a.n_states);
  ProfScope prof(K_GATE_UP, s);
  if (w_dtype == 1) {
    SD_NCH_DISPATCH(a.d, gate_up_kernel<bf16_t, NCH><<<grid, kThreads, lds, s>>>(
        a.x, a.norm, a.eps, a.norm != nullptr, (const bf16_t*)a.w_gate, (const bf16_t*)a.w_up,
        a.d, a.dff, a.t, a.gate_in, a.store_abs, a.act, a.keep, a.hmid, a.zero_buf, a.zero_n));
  } else {
    SD_NCH_DISPATCH(a.d, gate_up_kernel<float, NCH><<<grid, kThreads, lds, s>>>(
        a.x, a.norm, a.eps, a.norm != nullptr, (const float*)a.w_gate, (const float*)a.w_up,
        a.d, a.dff, a.t, a.gate_in, a.store_abs, a.act, a.keep, a.hmid, a.zero_buf, a.zero_n));
  }
}

}  // namespace sd
