// Streaming-read ceiling.  One plain pass over a device buffer with the
// access pattern of the library's weight streams (16-byte non-temporal loads,
// eight per wave in flight together, the waves in flight reading one
// contiguous window of the buffer), reduced to one XOR checksum per
// workgroup so that no load is dead.  The benchmark times it over 4 GiB and
// quotes the kernels' bandwidths against it as well as against the peak.
#include "common.hpp"
#include "internal.hpp"

namespace sd {

constexpr int kStreamThreads = 256;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(
    const u32x4* __restrict__ p, size_t n_chunks, unsigned* __restrict__ out) {
  __shared__ unsigned red[kStreamThreads / kWave];
  const int lane = lane_id(), wave_in = threadIdx.x / kWave;
  const size_t wave = (size_t)blockIdx.x * (kStreamThreads / kWave) + wave_in;
  const size_t n_waves = (size_t)gridDim.x * (kStreamThreads / kWave);
  u32x4 acc = u32x4{0u, 0u, 0u, 0u};
  // chunk c: 8 KB, 16-byte words [512 c, 512 c + 512): lane l loads words
  // 512 c + 64 k + l, k < 8
  for (size_t c = wave; c < n_chunks; c += n_waves) {
    const u32x4* q = p + c * 512 + lane;
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(q + 64 * k);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k];
  }
  unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o);
  if (lane == 0) red[wave_in] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned t = 0u;
#pragma unroll
    for (int w = 0; w < kStreamThreads / kWave; ++w) t ^= red[w];
    out[blockIdx.x] = t;
  }
}

void launch_stream_read(const void* buf, size_t bytes, unsigned* out, hipStream_t s) {
  launch_kernel(-1, stream_read_kernel, dim3(SD_STREAM_BLOCKS), dim3(kStreamThreads), 0, s,
                static_cast<const u32x4*>(buf), bytes / 8192, out);
}

}  // namespace sd
