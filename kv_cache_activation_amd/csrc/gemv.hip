// Weight-streaming GEMV kernels of the decode step (gfx950, wave64).
//
// Every kernel here reads one weight matrix once per step, the fixed term of
// the byte account in "Where Activation Sparsity and KV-Cache Sparsity Cross
// in LLM Decoding" (§1, §3.2).  Layout of the work, chosen by measurement on
// MI355X (one wave per weight row, rows dealt out across the whole grid so
// that the waves in flight together read one contiguous window of the matrix,
// which streams close to a plain sequential read):
//   * a workgroup stages the input vector in LDS once (times the norm
//     weights when there is a norm) and reduces sum(x^2) for the RMSNorm scale
//     rs, applied to each dot product at the end (RMSNorm(x) . w =
//     rs * (x * norm) . w), so the norm costs no extra pass over HBM; the
//     first weight rows are already in flight while it does so;
//   * a wave owns rows wave, wave + W, wave + 2W, ... (W = waves in the grid)
//     and streams each with 16-byte loads, the next row's loads issued before
//     the current row's arithmetic, reducing each dot product across the wave.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace sd {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

// Stage x (times nw when given) into LDS xs[0..d); returns the RMSNorm scale
// 1/sqrt(mean(x^2) + eps) when `norm`, else 1.  Every thread of the workgroup
// must call it (it holds a workgroup barrier).
__device__ float stage_x(const float* __restrict__ x, const float* __restrict__ nw, int d,
                         float eps, bool norm, float* xs) {
  __shared__ float red[kWavesPerBlock];
  float ss = 0.f;
  for (int i = 4 * threadIdx.x; i < d; i += 4 * kThreads) {  // d % 8 == 0
    float4 v = *reinterpret_cast<const float4*>(x + i);
    ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
    if (nw) {
      const float4 w = *reinterpret_cast<const float4*>(nw + i);
      v.x *= w.x; v.y *= w.y; v.z *= w.z; v.w *= w.w;
    }
    *reinterpret_cast<float4*>(xs + i) = v;
  }
  ss = wave_sum(ss);
  if (lane_id() == 0) red[threadIdx.x / kWave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) tot += red[w];
  return norm ? 1.0f / sqrtf(tot / (float)d + eps) : 1.0f;
}

// One weight row held by a wave: lane l holds the 16-byte chunks 8(l + 64k) .. +8.
template <typename WT, int NCH>
struct Row {
  Vec8<WT> w[NCH];
  __device__ __forceinline__ void load(const WT* __restrict__ W, int ld, int row, int d8) {
    const int lane = lane_id();
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int c8 = lane + kWave * k;
      if (c8 < d8) w[k].load(W + (size_t)row * ld + 8 * c8);
    }
  }
  // Full dot product with the LDS vector xs (every lane gets it).
  __device__ __forceinline__ float dot(const float* xs, int d8) const {
    const int lane = lane_id();
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int c8 = lane + kWave * k;
      if (c8 < d8) {
        float f[8], xv[8];
        w[k].to_float(f);
        load8f(xs + 8 * c8, xv);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(f[e], xv[e], acc);
      }
    }
    return wave_sum(acc);
  }
};

// ------------------------------------------------------------------ QKV
// x = RMSNorm(h) * attn_norm; [q; k; v] = W_qkv x; RoPE on q and k with the
// rotation table `rope` (cos and sin of pos * theta^(-2i/d_h) per pair index i,
// rotate-half pairs (i, i + d_h/2); the host computes it in double precision,
// since pos reaches 1e5+ and float angles would be off by 1e-2 rad, and an
// identity table turns RoPE off); q goes to q_out, k and v are
// rounded to the cache type and written at row row_full of the full cache and,
// when k_sel is given, at row row_sel of the gathered buffer.  A wave computes
// both rows of one rotation pair.
template <typename WT, typename KT, int NCH>
__global__ __launch_bounds__(kThreads) void qkv_rope_append_kernel(
    const float* __restrict__ h, const float* __restrict__ nw, float eps,
    const WT* __restrict__ W, int d, int h_q, int h_kv, int dh, RopeTable rope,
    float* __restrict__ q_out, KT* __restrict__ k_full, KT* __restrict__ v_full, int cap_full,
    int row_full, KT* __restrict__ k_sel, KT* __restrict__ v_sel, int cap_sel, int row_sel) {
  const int half = dh >> 1;
  const int d8 = d >> 3;
  const int n_pairs = (h_q + 2 * h_kv) * half;
  const int wave = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  const int n_waves = gridDim.x * kWavesPerBlock;
  extern __shared__ float xs[];
  Row<WT, NCH> ra, rb;
  int p = wave;
  if (p < n_pairs) {  // first pair's rows in flight during the staging
    const int head = p / half, i = p - head * half;
    ra.load(W, d, head * dh + i, d8);
    rb.load(W, d, head * dh + i + half, d8);
  }
  const float rs = stage_x(h, nw, d, eps, true, xs);
  if (p >= n_pairs) return;  // wave-uniform, after the workgroup barrier

  for (; p < n_pairs; p += n_waves) {
    const int head = p / half, i = p - head * half;
    float a = ra.dot(xs, d8) * rs;
    float b = rb.dot(xs, d8) * rs;
    const int pn = p + n_waves;
    if (pn < n_pairs) {  // next pair's rows in flight during the stores below
      const int hn = pn / half, in = pn - hn * half;
      ra.load(W, d, hn * dh + in, d8);
      rb.load(W, d, hn * dh + in + half, d8);
    }
    if (lane_id() == 0) {
      if (head < h_q + h_kv) {  // rotate q and k, not v
        const float c = rope.c[i], sn = rope.s[i];
        const float ra_ = a * c - b * sn;
        const float rb_ = b * c + a * sn;
        a = ra_;
        b = rb_;
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
          const size_t offs = ((size_t)kv * cap_sel + row_sel) * dh + i;
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
  const int d8 = din >> 3;
  const int wave = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  const int n_waves = gridDim.x * kWavesPerBlock;
  extern __shared__ float xs[];
  // h[row] is loaded before the row's weights, so waiting for it never waits
  // for a prefetch issued later
  const int lane = lane_id();
  Row<WT, NCH> r0, r1;
  float hc = 0.f;
  if (wave < dout) {
    if (lane == 0) hc = h[wave];
    r0.load(W, din, wave, d8);
  }
  stage_x(attn, nullptr, din, 0.f, false, xs);
  if (wave >= dout) return;  // wave-uniform, after the workgroup barrier
  int r = wave;
  for (;;) {
    const int rn = r + n_waves;
    float hn = 0.f;
    if (rn < dout) {
      if (lane == 0) hn = h[rn];
      r1.load(W, din, rn, d8);
    }
    const float s0 = r0.dot(xs, d8);
    if (lane == 0) h[r] = hc + s0;
    if (rn >= dout) break;
    const int rnn = rn + n_waves;
    if (rnn < dout) {
      if (lane == 0) hc = h[rnn];
      r0.load(W, din, rnn, d8);
    }
    const float s1 = r1.dot(xs, d8);
    if (lane == 0) h[rn] = hn + s1;
    if (rnn >= dout) break;
    r = rnn;
  }
}

// ------------------------------------------------------------------ CATS gate + up
// x = RMSNorm(h) * mlp_norm (or x itself without norm); a_i = SiLU(W_gate[i] . x)
// (or a_i read from `act` when gate_in); channel i is kept iff t < 0 or
// |a_i| > t; for kept channels hmid_i = a_i (W_up[i] . x): the up row is read
// only for kept channels.  keep[i] is 1 or 0.  With W_up == nullptr only `act`
// is produced (|a| when store_abs; calibration over blockIdx.y states).
// Two row buffers per wave: the next gate row streams in while the current
// channel's up row (if kept) is read into the buffer the gate row just left.
template <typename WT, int NCH, bool CALIB>
__global__ __launch_bounds__(kThreads) void gate_up_kernel(
    const float* __restrict__ xin, const float* __restrict__ nw, float eps, int norm,
    const WT* __restrict__ Wg, const WT* __restrict__ Wu, int d, int dff, float t, int gate_in,
    int store_abs, float* __restrict__ act, uint8_t* __restrict__ keep,
    float* __restrict__ hmid) {
  xin += (size_t)blockIdx.y * d;
  act += (size_t)blockIdx.y * dff;
  const int d8 = d >> 3;
  const int lane = lane_id();
  const int wave = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  const int n_waves = gridDim.x * kWavesPerBlock;
  extern __shared__ float xs[];
  Row<WT, NCH> ra, rb;
  if (wave < dff && !gate_in) ra.load(Wg, d, wave, d8);  // in flight during the staging
  const float rs = stage_x(xin, norm ? nw : nullptr, d, eps, norm != 0, xs);
  if (wave >= dff) return;  // wave-uniform, after the workgroup barrier

  // channel r with its gate row in `cur`; the next gate row goes into `nxt`
  auto channel = [&](Row<WT, NCH>& cur, Row<WT, NCH>& nxt, int r) {
    const int rn = r + n_waves;
    float a;
    if (gate_in) {
      a = act[r];
    } else {
      if (rn < dff) nxt.load(Wg, d, rn, d8);
      a = silu(cur.dot(xs, d8) * rs);
      if (lane == 0) act[r] = store_abs ? fabsf(a) : a;
    }
    if (!CALIB) {
      const bool k = t < 0.f || fabsf(a) > t;  // wave-uniform
      if (lane == 0) keep[r] = k;
      if (k) {
        cur.load(Wu, d, r, d8);
        const float u = cur.dot(xs, d8) * rs;
        if (lane == 0) hmid[r] = a * u;
      }
    }
  };
#pragma unroll 1
  for (int r = wave; r < dff; r += 2 * n_waves) {
    channel(ra, rb, r);
    if (r + n_waves >= dff) break;
    channel(rb, ra, r + n_waves);
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

// Grid of a row-streaming kernel: at most max_blocks workgroups, and no more
// waves than rows.
static int gemv_grid(int rows, int max_blocks) {
  const int need = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
  return need < max_blocks ? need : max_blocks;
}

template <typename WT, typename KT>
static void qkv_typed(const QkvArgs& a, hipStream_t s) {
  // one rotation pair per wave (all of a wave's rows in flight at once)
  const int grid = gemv_grid((a.h_q + 2 * a.h_kv) * a.dh / 2, 1024);
  const size_t lds = (size_t)a.d * sizeof(float);
  SD_NCH_DISPATCH(a.d, launch_kernel(K_QKV, qkv_rope_append_kernel<WT, KT, NCH>, dim3(grid),
                                      dim3(kThreads), (uint32_t)lds, s, a.h, a.norm, a.eps,
                                      (const WT*)a.w, a.d, a.h_q, a.h_kv, a.dh, a.rope, a.q_out,
                                      (KT*)a.k_full, (KT*)a.v_full, a.cap_full, a.row_full,
                                      (KT*)a.k_sel, (KT*)a.v_sel, a.cap_sel, a.row_sel));
}

void launch_qkv(const QkvArgs& a, int w_dtype, int kv_dtype, hipStream_t s) {
  if (w_dtype == 1 && kv_dtype == 1) qkv_typed<bf16_t, bf16_t>(a, s);
  else if (w_dtype == 1) qkv_typed<bf16_t, float>(a, s);
  else if (kv_dtype == 1) qkv_typed<float, bf16_t>(a, s);
  else qkv_typed<float, float>(a, s);
}

void launch_o(const float* attn, const void* w, int din, int dout, float* h, int w_dtype,
              hipStream_t s) {
  const int grid = gemv_grid(dout, 1024);  // one row per wave for 4096 rows (measured best)
  const size_t lds = (size_t)din * sizeof(float);
  if (w_dtype == 1) {
    SD_NCH_DISPATCH(din, launch_kernel(K_O, o_residual_kernel<bf16_t, NCH>, dim3(grid),
                                       dim3(kThreads), (uint32_t)lds, s, attn, (const bf16_t*)w,
                                       din, dout, h));
  } else {
    SD_NCH_DISPATCH(din, launch_kernel(K_O, o_residual_kernel<float, NCH>, dim3(grid),
                                       dim3(kThreads), (uint32_t)lds, s, attn, (const float*)w,
                                       din, dout, h));
  }
}

void launch_gate_up(const GateUpArgs& a, int w_dtype, hipStream_t s) {
  dim3 grid(gemv_grid(a.dff, 1024), a.n_states);
  const size_t lds = (size_t)a.d * sizeof(float);
  // the calibration instance (no up projection) has a kernel name of its own
#define SD_GATE_UP(T, CAL)                                                                    \
  SD_NCH_DISPATCH(a.d, launch_kernel(K_GATE_UP, gate_up_kernel<T, NCH, CAL>, grid,            \
                                     dim3(kThreads), (uint32_t)lds, s, a.x, a.norm, a.eps,    \
                                     (int)(a.norm != nullptr), (const T*)a.w_gate,            \
                                     (const T*)a.w_up, a.d, a.dff, a.t, a.gate_in,            \
                                     a.store_abs, a.act, a.keep, a.hmid))
  const bool calib = a.w_up == nullptr;
  if (w_dtype == 1) {
    if (calib) {
      SD_GATE_UP(bf16_t, true);
    } else {
      SD_GATE_UP(bf16_t, false);
    }
  } else {
    if (calib) {
      SD_GATE_UP(float, true);
    } else {
      SD_GATE_UP(float, false);
    }
  }
#undef SD_GATE_UP
}

}  // namespace sd
