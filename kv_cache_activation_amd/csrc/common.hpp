// Device helpers shared by the gfx950 kernels of the sparse decode step.
//
// Everything here is wave64 CDNA code: lane groups of 16 (a DPP "row") are the
// unit of the small dot-product reductions, 16-byte global loads are the unit
// of HBM traffic, and bf16 is widened to float32 by a shift (its bits are the
// upper half of a float32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sd {

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- widening
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bfloat16, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// ---------------------------------------------------------------- cross-workgroup
// Agent-scope (device-coherent) stores and loads of float32 partial sums that
// one workgroup writes and another, possibly on another XCD, reads after a
// ticket: the stores are written through to memory, the loads bypass the
// XCD-local caches.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<unsigned*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_agent(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<unsigned*>(const_cast<float*>(p)),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// p[0] + p[stride] + ... + p[(n - 1) stride], added in index order, loaded at
// agent scope sixteen at a time: the compiler keeps atomic loads in program
// order and waits for each before its add, so a plain loop would pay one
// memory round trip per term.
__device__ __forceinline__ float sum_agent(const float* p, size_t stride, int n) {
  float v = 0.f;
  for (int k0 = 0; k0 < n; k0 += 16) {
    float t[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) t[k] = k0 + k < n ? load_agent(p + (size_t)(k0 + k) * stride) : 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) v += t[k];  // terms past n add +0
  }
  return v;
}

// ---------------------------------------------------------------- RoPE
// cos and sin of the rotation of pair (i, i + d_h / 2) at position pos:
// angle pos * theta^(-2 i / d_h), formed in double precision.
__device__ __forceinline__ void rope_cs(int pos, int i, int dh, float theta, float& c, float& s) {
  const double inv = pow((double)theta, -2.0 * (double)i / (double)dh);
  const double ang = (double)pos * inv;
  c = (float)cos(ang);
  s = (float)sin(ang);
}

// ---------------------------------------------------------------- matrix cores
// Operand type of v_mfma_f32_16x16x32_bf16 (eight bf16 values per lane).
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Eight float32 values as three bf16 parts, hi + mid + lo == x: hi carries
// the top 8 significand bits, mid the next 8 (x - hi is exact in float32),
// lo the rest.  Products of a part with a bf16 value are exact in float32, so
// a matrix-core sum over the three parts keeps float32 accuracy.
__device__ __forceinline__ void split3_bf16(const float (&x)[8], u32x4& hi, u32x4& mid,
                                            u32x4& lo) {
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t hh[2], mm[2], ll[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float v = x[2 * p + e];
      const bf16_t bh = f32_to_bf16(v);
      const float r1 = v - bf16_lo((uint32_t)bh);
      const bf16_t bm = f32_to_bf16(r1);
      hh[e] = bh;
      mm[e] = bm;
      ll[e] = f32_to_bf16(r1 - bf16_lo((uint32_t)bm));
    }
    h[p] = hh[0] | (hh[1] << 16);
    m[p] = mm[0] | (mm[1] << 16);
    l[p] = ll[0] | (ll[1] << 16);
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  mid = u32x4{m[0], m[1], m[2], m[3]};
  lo = u32x4{l[0], l[1], l[2], l[3]};
}

// Eight consecutive elements of a row as float32, from one 16-byte load
// (bf16) or two (float32).  p must be 16-byte aligned.
template <typename T> struct Vec8;

template <> struct Vec8<bf16_t> {
  u32x4 raw;
  __device__ __forceinline__ void load(const bf16_t* p) {
    raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  __device__ __forceinline__ void load_cached(const bf16_t* p) {
    raw = *reinterpret_cast<const u32x4*>(p);
  }
  __device__ __forceinline__ void to_float(float (&f)[8]) const {
    f[0] = bf16_lo(raw.x); f[1] = bf16_hi(raw.x);
    f[2] = bf16_lo(raw.y); f[3] = bf16_hi(raw.y);
    f[4] = bf16_lo(raw.z); f[5] = bf16_hi(raw.z);
    f[6] = bf16_lo(raw.w); f[7] = bf16_hi(raw.w);
  }
};

template <> struct Vec8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
  }
  __device__ __forceinline__ void load_cached(const float* p) {
    a = reinterpret_cast<const f32x4*>(p)[0];
    b = reinterpret_cast<const f32x4*>(p)[1];
  }
  __device__ __forceinline__ void to_float(float (&f)[8]) const {
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

__device__ __forceinline__ void store8(float* p, const float (&f)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
}

__device__ __forceinline__ void load8f(const float* p, float (&f)[8]) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// Store one element of a cache row, rounded to the cache type.
__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_elem(bf16_t* p, float v) { *p = f32_to_bf16(v); }

// ---------------------------------------------------------------- reductions
// DPP controls (GCN/CDNA encoding).
constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LANES lanes (4, 8 or 16); every lane gets the sum.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LANES == 4 || LANES == 8 || LANES == 16, "group of 4, 8 or 16 lanes");
  x += dpp<kDppQuadSwap1>(x);
  x += dpp<kDppQuadSwap2>(x);
  if (LANES >= 8) x += dpp<kDppRowHalfMirror>(x);
  if (LANES >= 16) x += dpp<kDppRowMirror>(x);
  return x;
}

template <int LANES>
__device__ __forceinline__ float group_max(float x) {
  static_assert(LANES == 4 || LANES == 8 || LANES == 16, "group of 4, 8 or 16 lanes");
  x = fmaxf(x, dpp<kDppQuadSwap1>(x));
  x = fmaxf(x, dpp<kDppQuadSwap2>(x));
  if (LANES >= 8) x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  if (LANES >= 16) x = fmaxf(x, dpp<kDppRowMirror>(x));
  return x;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// x of lane l ^ OFF (OFF = 8, 16 or 32), with VALU lane exchanges only: a
// DPP row rotation by 8 (within a row of 16 lanes it is the xor by 8), and
// gfx950's permlane swaps for rows and half-waves (each swap exchanges the
// odd rows / upper half of one operand with the even rows / lower half of
// the other, so swapping x with itself gives each lane its partner in one of
// the two results).  An LDS permute per exchange costs a round trip through
// the LDS unit instead; this is on the path of every dot-product reduction.
template <int OFF>
__device__ __forceinline__ float xor_lanes(float x) {
  static_assert(OFF == 8 || OFF == 16 || OFF == 32, "xor by 8, 16 or 32");
  if constexpr (OFF == 8) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
  } else if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((lane_id() & 16) ? r[0] : r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((lane_id() & 32) ? r[0] : r[1]);
  }
}

// Full-wave sum and max (every lane gets the result).
__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  x += xor_lanes<16>(x);
  x += xor_lanes<32>(x);
  return x;
}

__device__ __forceinline__ int wave_sum_int(int x) {
  for (int off = 1; off < kWave; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

// Inclusive prefix sum over the wave's lanes (DPP row shifts, then row
// broadcasts of lanes 15 and 31 into the following rows).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  x = group_max<16>(x);
  x = fmaxf(x, xor_lanes<16>(x));
  x = fmaxf(x, xor_lanes<32>(x));
  return x;
}


__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Stage x (times nw when given) into LDS xs[0..d) with a workgroup of THREADS
// threads; returns the RMSNorm scale 1/sqrt(mean(x^2) + eps) when `norm`, else
// 1.  Every thread of the workgroup must call it (it holds a workgroup
// barrier).  d % 4 == 0 and x, nw 16-byte aligned.
template <int THREADS>
__device__ float stage_x(const float* __restrict__ x, const float* __restrict__ nw, int d,
                         float eps, bool norm, float* xs) {
  constexpr int kWaves = THREADS / kWave;
  __shared__ float red[kWaves];
  float ss = 0.f;
  for (int i = 4 * threadIdx.x; i < d; i += 4 * THREADS) {
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
  for (int w = 0; w < kWaves; ++w) tot += red[w];
  return norm ? 1.0f / sqrtf(tot / (float)d + eps) : 1.0f;
}

// stage_x in two halves, so the input's loads can be issued before the first
// weight rows and the workgroup's staging waits only for them: load() reads
// this thread's float4 chunks 4(t + THREADS k) of x (and nw) into registers,
// finish() reduces sum(x^2), writes x * nw to LDS and holds the barrier.
// d <= 4 NV THREADS; FULL: d == 4 NV THREADS (no bounds tests); NW: nw is
// given (the loads then have no branch around them either).
template <int THREADS, int NV, bool FULL, bool NW>
struct XStage {
  float4 x[NV], w[NV];
  __device__ __forceinline__ void load(const float* __restrict__ xin,
                                       const float* __restrict__ nw, int d) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int i = 4 * (threadIdx.x + THREADS * k);
      x[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      w[k] = make_float4(1.f, 1.f, 1.f, 1.f);
      if (FULL || i < d) {
        x[k] = *reinterpret_cast<const float4*>(xin + i);
        if (NW) w[k] = *reinterpret_cast<const float4*>(nw + i);
      }
    }
  }
  __device__ __forceinline__ float finish(int d, float eps, bool norm, float* xs) {
    constexpr int kWaves = THREADS / kWave;
    __shared__ float red[kWaves];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int i = 4 * (threadIdx.x + THREADS * k);
      const float4 v = x[k];
      ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
      if (FULL || i < d)
        *reinterpret_cast<float4*>(xs + i) =
            make_float4(v.x * w[k].x, v.y * w[k].y, v.z * w[k].z, v.w * w[k].w);
    }
    ss = wave_sum(ss);
    if (lane_id() == 0) red[threadIdx.x / kWave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) tot += red[v];
    return norm ? 1.0f / sqrtf(tot / (float)d + eps) : 1.0f;
  }
};

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
  // All NCH chunks, no bounds test (d == 512 NCH): with no branch around the
  // loads the compiler can wait for exactly this row's loads later instead of
  // for every load in flight.
  __device__ __forceinline__ void load_full(const WT* __restrict__ W, int ld, int row) {
    const int lane = lane_id();
#pragma unroll
    for (int k = 0; k < NCH; ++k) w[k].load(W + (size_t)row * ld + 8 * (lane + kWave * k));
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
  // dot() for d == 512 NCH (no bounds tests)
  __device__ __forceinline__ float dot_full(const float* xs) const {
    const int lane = lane_id();
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      float f[8], xv[8];
      w[k].to_float(f);
      load8f(xs + 8 * (lane + kWave * k), xv);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(f[e], xv[e], acc);
    }
    return wave_sum(acc);
  }
};

// Chunks of 8 columns a row of d (d % 8 == 0) elements needs per lane, as a
// power of two (the template argument NCH of Row).
inline int nch_for(int d) {
  int need = (d / 8 + kWave - 1) / kWave;
  int n = 1;
  while (n < need) n <<= 1;
  return n;
}

#define SD_NCH_DISPATCH(D, ...)                                  \
  switch (::sd::nch_for(D)) {                                    \
    case 1: { constexpr int NCH = 1; __VA_ARGS__; } break;   \
    case 2: { constexpr int NCH = 2; __VA_ARGS__; } break;   \
    case 4: { constexpr int NCH = 4; __VA_ARGS__; } break;   \
    case 8: { constexpr int NCH = 8; __VA_ARGS__; } break;   \
    default: { constexpr int NCH = 16; __VA_ARGS__; } break; \
  }

}  // namespace sd
