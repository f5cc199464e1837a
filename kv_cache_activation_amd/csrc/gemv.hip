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

#include <map>
#include <mutex>
#include <utility>

#include "common.hpp"
#include "internal.hpp"

namespace sd {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
// Workgroup size of the d = 4096 instances with bf16 weights.  Measured on
// MI355X (32-layer composed step at 131072 context): 512 threads for O, one
// row per wave, two workgroups per unit, each staging its 16 KB input once
// per 8 rows (1024 threads: 7.0 against 8.2 us per launch for 256; 512: the
// step 2485-2487 against 2495-2499 us for 1024); QKV and gate + up were no
// faster with wider workgroups.
constexpr int kQkvWide = kThreads, kOWide = 512, kGateWide = kThreads;
// QKV workgroups per compute unit, at most: with one, each unit stages the
// input once and its four waves take more rows each.  Measured in the
// composed step at 131072 context: 2483-2484 us per step against 2494-2496
// with the three the occupancy allows (2486-2489 with two, 2505 with 384
// workgroups); gate + up was slower with fewer workgroups (2511 with 768,
// 2541 with 512, against 2506 with 1024).
constexpr int kQkvPerCu = 1;

// float4 chunks per thread when T threads stage a row of 512 NCH elements
// (EXACT: no bounds tests)
template <int T, int NCH>
struct StageNV {
  static constexpr int NV = (NCH * 128 + T - 1) / T;
  static constexpr bool EXACT = (NCH * 128) % T == 0;
};

// Full dot product of a row with the LDS copy of x (every lane gets it).
// FULL: d == 512 NCH.
template <bool FULL, typename WT, int NCH>
__device__ __forceinline__ float row_dot(const Row<WT, NCH>& r, const float* xs, int d8) {
  return FULL ? r.dot_full(xs) : r.dot(xs, d8);
}

template <bool FULL, typename WT, int NCH>
__device__ __forceinline__ void load_row(Row<WT, NCH>& r, const WT* __restrict__ W, int ld,
                                         int row, int d8) {
  if constexpr (FULL) r.load_full(W, ld, row);
  else r.load(W, ld, row, d8);
}

// Streams the n rows row_of(0), row_of(1), ... of W (1 <= n <= 64) through
// the calling wave with two rows in flight and returns in lane k the dot
// product of row k with x (LDS copy xs); `ra` already holds row 0.  What
// keeps the loads flowing, measured on MI355X (117 MB gate matrix: 25.6 ->
// 20.9 us):
//  * the loop body issues the next row's loads with no branch around them
//    (the last row is peeled off, and full-width rows have no bounds tests),
//    so the compiler waits for exactly the older row's loads instead of for
//    every load in flight;
//  * x is read from LDS for every row: an empty asm with a memory clobber
//    stops the compiler from hoisting those reads into 64 more VGPRs, which
//    would cost a wave per SIMD of occupancy;
//  * results stay in registers until the caller stores them after the loop
//    (a store in the loop shares the loads' completion counter).
template <bool FULL, typename WT, int NCH, typename RowOf>
__device__ __forceinline__ float stream_rows(const WT* __restrict__ W, int ld, int d8, int n,
                                             const float* xs, Row<WT, NCH>& ra,
                                             Row<WT, NCH>& rb, RowOf row_of) {
  const int lane = lane_id();
  float mine = 0.f;
  auto take = [&](const Row<WT, NCH>& r, int k) {
    asm volatile("" ::: "memory");
    const float s = row_dot<FULL>(r, xs, d8);
    if (lane == k) mine = s;
  };
  int k = 0;
#pragma unroll 1
  for (; k + 2 < n; k += 2) {
    load_row<FULL>(rb, W, ld, row_of(k + 1), d8);
    take(ra, k);
    load_row<FULL>(ra, W, ld, row_of(k + 2), d8);
    take(rb, k + 1);
  }
  if (k + 1 < n) {
    load_row<FULL>(rb, W, ld, row_of(k + 1), d8);
    take(ra, k);
    take(rb, k + 1);
  } else {
    take(ra, k);
  }
  return mine;
}

// ------------------------------------------------------------------ QKV
// x = RMSNorm(h) * attn_norm; [q; k; v] = W_qkv x; RoPE on q and k with the
// rotation table `rope` (cos and sin of pos * theta^(-2i/d_h) per pair index i,
// rotate-half pairs (i, i + d_h/2); the host computes it in double precision,
// since pos reaches 1e5+ and float angles would be off by 1e-2 rad, and an
// identity table turns RoPE off); q goes to q_out, k and v are
// rounded to the cache type and written at row row_full of the full cache and,
// when k_sel is given, at row row_sel of the gathered buffer.  A wave computes
// both rows of the rotation pairs wave, wave + W, ... (W waves in the grid,
// at most 32 pairs per wave); lane j then rotates and stores its j-th pair.
template <typename WT, typename KT, int NCH, bool FULL, int T>
__global__ __launch_bounds__(T) void qkv_rope_append_kernel(
    const float* __restrict__ h, const float* __restrict__ nw, float eps,
    const WT* __restrict__ W, int d, int h_q, int h_kv, int dh, RopeTable rope,
    float* __restrict__ q_out, KT* __restrict__ k_full, KT* __restrict__ v_full, int cap_full,
    int row_full, KT* __restrict__ k_sel, KT* __restrict__ v_sel, int cap_sel, int row_sel,
    int ragged, HeadInts sel_rows) {
  const int half = dh >> 1;
  const int d8 = d >> 3;
  const int n_pairs = (h_q + 2 * h_kv) * half;
  const int wave = blockIdx.x * (T / kWave) + threadIdx.x / kWave;
  const int n_waves = gridDim.x * (T / kWave);
  const int lane = lane_id();
  const int my_pairs = wave < n_pairs ? (n_pairs - wave + n_waves - 1) / n_waves : 0;
  // the epilogue's inputs now, not after the dot products: the output
  // pointers, and lane j's rotation angle (pair wave + j W) and gathered row
  asm volatile("" ::"s"(q_out), "s"(k_full), "s"(v_full), "s"(k_sel), "s"(v_sel));
  const int ep = wave + (lane < my_pairs ? lane : 0) * n_waves;
  const int ep_head = ep / half, ep_i = ep - ep_head * half;
  const float ep_c = rope.c[ep_i], ep_s = rope.s[ep_i];
  const int ep_kv = ep_head < h_q + h_kv ? ep_head - h_q : ep_head - h_q - h_kv;
  const int ep_rsel = ragged ? sel_rows.v[ep_kv & (kMaxKvHeads - 1)] : row_sel;
  // row k of this wave: pair wave + (k / 2) W, first (k even) or second row
  auto row_of = [&](int k) {
    const int p = wave + (k >> 1) * n_waves;
    const int head = p / half, i = p - head * half;
    return head * dh + i + (k & 1) * half;
  };
  extern __shared__ float xs[];
  XStage<T, StageNV<T, NCH>::NV, FULL && StageNV<T, NCH>::EXACT, true> st;
  st.load(h, nw, d);  // x first: the staging then waits for it alone
  // the first pair's rows are in flight during the staging (a wave without
  // pairs, only when waves outnumber pairs, reads pair 0 and drops it: no
  // branch around the loads)
  Row<WT, NCH> ra, rb;
  {
    const int p0 = my_pairs > 0 ? wave : 0;
    const int head = p0 / half, i = p0 - head * half;
    load_row<FULL>(ra, W, d, head * dh + i, d8);
    load_row<FULL>(rb, W, d, head * dh + i + half, d8);
  }
  const float rs = st.finish(d, eps, true, xs);
  if (my_pairs == 0) return;  // wave-uniform, after the workgroup barrier
  // rows 0 and 1 are both in flight: take them first, then stream the rest
  const float s0 = row_dot<FULL>(ra, xs, d8), s1 = row_dot<FULL>(rb, xs, d8);
  float mine = lane == 0 ? s0 : lane == 1 ? s1 : 0.f;
  const int n_rows = 2 * my_pairs;
  if (n_rows > 2) {
    load_row<FULL>(ra, W, d, row_of(2), d8);
    const float rest = stream_rows<FULL>(W, d, d8, n_rows - 2, xs, ra, rb,
                                         [&](int k) { return row_of(k + 2); });
    const float up = __shfl_up(rest, 2);
    if (lane >= 2) mine = up;
  }
  // lane j: rows 2j and 2j+1 of the wave
  const float a0 = __shfl(mine, 2 * lane) * rs;
  const float b0 = __shfl(mine, 2 * lane + 1) * rs;
  if (lane >= my_pairs) return;
  const int head = ep_head, i = ep_i;
  float a = a0, b = b0;
  if (head < h_q + h_kv) {  // rotate q and k, not v
    a = a0 * ep_c - b0 * ep_s;
    b = b0 * ep_c + a0 * ep_s;
  }
  if (head < h_q) {
    q_out[head * dh + i] = a;
    q_out[head * dh + i + half] = b;
  } else {
    const bool is_k = head < h_q + h_kv;
    const int kv = ep_kv;
    KT* full = is_k ? k_full : v_full;
    const size_t off = ((size_t)kv * cap_full + row_full) * dh + i;
    store_elem(full + off, a);
    store_elem(full + off + half, b);
    if (k_sel) {
      KT* sel = is_k ? k_sel : v_sel;  // ragged budgets: each KV head at its own row (ep_rsel)
      const size_t offs = ((size_t)kv * cap_sel + ep_rsel) * dh + i;
      store_elem(sel + offs, a);
      store_elem(sel + offs + half, b);
    }
  }
}

// ------------------------------------------------------------------ O
// h[r] += W_o[r] . attn  (residual add; attn is the attention output).  ONE:
// the grid has a wave per row (no second row buffer: more waves fit).
template <typename WT, int NCH, bool FULL, bool ONE, int T>
__global__ __launch_bounds__(T) void o_residual_kernel(const float* __restrict__ attn,
                                                              const WT* __restrict__ W, int din,
                                                              int dout, float* __restrict__ h) {
  const int d8 = din >> 3;
  const int wave = blockIdx.x * (T / kWave) + threadIdx.x / kWave;
  const int n_waves = gridDim.x * (T / kWave);
  const int lane = lane_id();
  const int n = wave < dout ? (dout - wave + n_waves - 1) / n_waves : 0;  // <= 64
  extern __shared__ float xs[];
  XStage<T, StageNV<T, NCH>::NV, FULL && StageNV<T, NCH>::EXACT, false> st;
  st.load(attn, nullptr, din);  // x first: the staging then waits for it alone
  // lane k's residual h[wave + k W] now, not after the dot products
  const float h_old = lane < n ? h[wave + lane * n_waves] : 0.f;
  Row<WT, NCH> ra, rb;  // rb unused (no registers) when ONE
  load_row<FULL>(ra, W, din, n > 0 ? wave : 0, d8);  // no branch around the loads
  st.finish(din, 0.f, false, xs);
  if (n == 0) return;  // wave-uniform, after the workgroup barrier
  float s;
  if constexpr (ONE) {
    s = row_dot<FULL>(ra, xs, d8);
  } else {
    s = stream_rows<FULL>(W, din, d8, n, xs, ra, rb, [&](int k) { return wave + k * n_waves; });
  }
  if (lane < n) h[wave + lane * n_waves] = h_old + s;
}

// ------------------------------------------------------------------ CATS gate (+ up)
// x = RMSNorm(h) * mlp_norm (NORM; x itself otherwise); a_i = SiLU(W_gate[i] . x)
// (or a_i read from `act` when gate_in); act[i] = a_i (|a_i| when store_abs);
// keep[i] = 1 iff t < 0 or |a_i| > t, else 0 (keep may be null).  The gate is
// dense in CATS: every row is read, so the first phase is a plain
// row-streaming GEMV over the wave's rows.  With W_up given, each wave then
// reads the up rows of its kept channels only, two at a time with both
// loads issued together, and writes hmid_i = a_i (W_up[i] . x), zero for a
// dropped channel.  blockIdx.y selects one
// of several input states (calibration); the calibration instance (CALIB)
// only has a kernel name of its own.
template <typename WT, int NCH, bool FULL, bool NORM, bool CALIB, int T>
__global__ __launch_bounds__(T) void gate_kernel(
    const float* __restrict__ xin, const float* __restrict__ nw, float eps,
    const WT* __restrict__ Wg, const WT* __restrict__ Wu, int d, int dff, float t, int gate_in,
    int store_abs, float* __restrict__ act, uint8_t* __restrict__ keep,
    float* __restrict__ hmid) {
  xin += (size_t)blockIdx.y * d;
  act += (size_t)blockIdx.y * dff;
  const int d8 = d >> 3;
  const int lane = lane_id();
  const int wave = blockIdx.x * (T / kWave) + threadIdx.x / kWave;
  const int n_waves = gridDim.x * (T / kWave);
  const int n = wave < dff ? (dff - wave + n_waves - 1) / n_waves : 0;  // <= 64
  extern __shared__ float xs[];
  XStage<T, StageNV<T, NCH>::NV, FULL && StageNV<T, NCH>::EXACT, NORM> st;
  st.load(xin, nw, d);  // x first: the staging then waits for it alone
  Row<WT, NCH> ra, rb;
  if (!gate_in) load_row<FULL>(ra, Wg, d, n > 0 ? wave : 0, d8);  // in flight during the staging
  const float rs = st.finish(d, eps, NORM, xs);
  if (n == 0) return;  // wave-uniform, after the workgroup barrier
  // lane k: channel wave + k W (k < n)
  const int r = wave + lane * n_waves;
  float a = 0.f;
  if (gate_in) {
    if (lane < n) a = act[r];
  } else {
    const float s = stream_rows<FULL>(Wg, d, d8, n, xs, ra, rb,
                                      [&](int k) { return wave + k * n_waves; });
    a = silu(s * rs);
  }
  const bool kept = lane < n && (t < 0.f || fabsf(a) > t);
  float hm = 0.f;
  if (!CALIB && Wu) {
    uint64_t km = __ballot(kept);  // wave-uniform
#pragma unroll 1
    while (km) {
      const int k0 = __ffsll((unsigned long long)km) - 1;
      km &= km - 1;
      const int k1 = km ? __ffsll((unsigned long long)km) - 1 : -1;
      if (k1 >= 0) km &= km - 1;
      load_row<FULL>(ra, Wu, d, wave + k0 * n_waves, d8);
      if (k1 >= 0) load_row<FULL>(rb, Wu, d, wave + k1 * n_waves, d8);
      asm volatile("" ::: "memory");  // x from LDS per row, as in stream_rows
      const float u0 = row_dot<FULL>(ra, xs, d8) * rs;
      if (lane == k0) hm = a * u0;
      if (k1 >= 0) {
        asm volatile("" ::: "memory");
        const float u1 = row_dot<FULL>(rb, xs, d8) * rs;
        if (lane == k1) hm = a * u1;
      }
    }
  }
  if (lane < n) {
    if (!gate_in) act[r] = store_abs ? fabsf(a) : a;
    if (!CALIB && keep) keep[r] = kept;
    if (!CALIB && Wu) hmid[r] = hm;  // zero for a dropped channel
  }
}

// ------------------------------------------------------------------ launchers
// Grid of a row-streaming kernel: as many workgroups as the chip holds at
// once (compute units x resident workgroups per unit, which the kernel's
// register use decides, at most cap_per_cu when that is positive), no more
// waves than work items, and at most per_wave items per wave (a wave keeps
// one result per lane).
template <int T, typename K>
static int gemv_grid(K kernel, int rows, int per_wave, size_t lds, int cap_per_cu) {
  constexpr int kWavesPerBlock = T / kWave;
  // resident workgroups per compute unit, per kernel and LDS size (queried once)
  static std::mutex mu;
  static std::map<std::pair<const void*, size_t>, int> cache;
  int per_cu = 0;
  {
    std::lock_guard<std::mutex> g(mu);
    const auto key = std::make_pair(reinterpret_cast<const void*>(kernel), lds);
    auto it = cache.find(key);
    if (it == cache.end()) {
      int nb = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, T, lds) != hipSuccess ||
          nb < 1)
        nb = 1;
      it = cache.emplace(key, nb).first;
    }
    per_cu = it->second;
  }
  if (cap_per_cu > 0 && per_cu > cap_per_cu) per_cu = cap_per_cu;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  int grid = cus * per_cu;
  const int need = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
  const int least = (rows + kWavesPerBlock * per_wave - 1) / (kWavesPerBlock * per_wave);
  if (grid > need) grid = need;
  if (grid < least) grid = least;
  return grid < 1 ? 1 : grid;
}

// SD_NCH_DISPATCH plus FULL = (the row width is exactly 512 NCH elements)
#define SD_ROW_DISPATCH(D, ...)                                                   \
  SD_NCH_DISPATCH(D, if ((D) == 512 * NCH) {                                     \
    constexpr bool FULL = true;                                                   \
    __VA_ARGS__;                                                                  \
  } else {                                                                        \
    constexpr bool FULL = false;                                                  \
    __VA_ARGS__;                                                                  \
  })

template <int T, typename K, typename... Args>
static void launch_rows(int kind, K kernel, int items, int per_wave, int grid_y, size_t lds,
                        int cap_per_cu, hipStream_t s, Args... args) {
  const int grid = gemv_grid<T>(kernel, items, per_wave, lds, cap_per_cu);
  launch_kernel(kind, kernel, dim3(grid, grid_y), dim3(T), (uint32_t)lds, s, args...);
}

template <typename WT, typename KT>
static void qkv_typed(const QkvArgs& a, hipStream_t s) {
  const int pairs = (a.h_q + 2 * a.h_kv) * a.dh / 2;
  const size_t lds = (size_t)a.d * sizeof(float);
  SD_ROW_DISPATCH(a.d, constexpr int TH = (NCH == 8 && FULL && sizeof(WT) == 2) ? kQkvWide : kThreads;
                  launch_rows<TH>(K_QKV, qkv_rope_append_kernel<WT, KT, NCH, FULL, TH>, pairs, kWave / 2,
                                   1, lds, kQkvPerCu, s, a.h, a.norm, a.eps,
                                      (const WT*)a.w, a.d, a.h_q, a.h_kv, a.dh, a.rope, a.q_out,
                                      (KT*)a.k_full, (KT*)a.v_full, a.cap_full, a.row_full,
                                      (KT*)a.k_sel, (KT*)a.v_sel, a.cap_sel, a.row_sel, a.ragged,
                                   a.sel_rows));
}

void launch_qkv(const QkvArgs& a, int w_dtype, int kv_dtype, hipStream_t s) {
  if (w_dtype == 1 && kv_dtype == 1) qkv_typed<bf16_t, bf16_t>(a, s);
  else if (w_dtype == 1) qkv_typed<bf16_t, float>(a, s);
  else if (kv_dtype == 1) qkv_typed<float, bf16_t>(a, s);
  else qkv_typed<float, float>(a, s);
}

void launch_o(const float* attn, const void* w, int din, int dout, float* h, int w_dtype,
              hipStream_t s) {
  const size_t lds = (size_t)din * sizeof(float);
  // a wave per row while that fits the grid limit, else streamed rows
  const bool one = dout <= 4096 * kWavesPerBlock;
#define SD_O(T, ONE_)                                                                          \
  SD_ROW_DISPATCH(din, constexpr int TH = (NCH == 8 && FULL && sizeof(T) == 2) ? kOWide : kThreads; \
                  launch_rows<TH>(K_O, o_residual_kernel<T, NCH, FULL, ONE_, TH>, dout,       \
                                   ONE_ ? 1 : kWave, 1, lds, 0, s, attn, (const T*)w, din, dout, h))
  if (w_dtype == 1) {
    if (one) {
      SD_O(bf16_t, true);
    } else {
      SD_O(bf16_t, false);
    }
  } else {
    if (one) {
      SD_O(float, true);
    } else {
      SD_O(float, false);
    }
  }
#undef SD_O
}

void launch_gate(const GateArgs& a, int w_dtype, hipStream_t s) {
  const size_t lds = (size_t)a.d * sizeof(float);
  // the calibration instance has a kernel name of its own
#define SD_GATE_N(T, NRM, CAL)                                                               \
  SD_ROW_DISPATCH(a.d, constexpr int TH = (NCH == 8 && FULL && sizeof(T) == 2) ? kGateWide : kThreads; \
                  launch_rows<TH>(K_GATE_UP, gate_kernel<T, NCH, FULL, NRM, CAL, TH>, a.dff, kWave, \
                                   a.n_states, lds, 0, s, a.x, a.norm, a.eps,                 \
                                   (const T*)a.w_gate, (const T*)a.w_up, a.d, a.dff, a.t,     \
                                   a.gate_in, a.store_abs, a.act, a.keep, a.hmid))
#define SD_GATE(T, CAL)          \
  if (a.norm) {                  \
    SD_GATE_N(T, true, CAL);     \
  } else {                       \
    SD_GATE_N(T, false, CAL);    \
  }
  if (w_dtype == 1) {
    if (a.calib) {
      SD_GATE(bf16_t, true);
    } else {
      SD_GATE(bf16_t, false);
    }
  } else {
    if (a.calib) {
      SD_GATE(float, true);
    } else {
      SD_GATE(float, false);
    }
  }
#undef SD_GATE
#undef SD_GATE_N
}

}  // namespace sd
