// sd_decode_step_noalloc: the decode step with its intermediate state in a
// buffer the library owns, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  Same kernels and launch order as sd_decode_step.
//
// The buffer is a file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Host code
// must not pass the array's name to a kernel (on the host it is only a
// stand-in symbol); the address each device gives for it is looked up once
// per device with hipGetSymbolAddress and kept.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/sd.h"
#include "internal.hpp"

namespace {

constexpr size_t kScratchBytes = SD_NOALLOC_SCRATCH_BYTES;  // 64 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch`, per device ordinal

sd_status scratch_of_current_device(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    char msg[160];
    snprintf(msg, sizeof msg, "sd_decode_step_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    return sd::set_error(SD_EHIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices)
    return sd::set_error(SD_EUNSUPPORTED, "sd_decode_step_noalloc: device ordinal above 63");
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r != hipSuccess || !p) {
      char msg[160];
      snprintf(msg, sizeof msg, "sd_decode_step_noalloc: hipGetSymbolAddress: %s",
               hipGetErrorString(r));
      return sd::set_error(SD_EHIP, msg);
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SD_OK;
}

}  // namespace

extern "C" sd_status sd_decode_step_noalloc(const sd_dims* dims, int32_t n_layers,
                                            sd_layer* layers, int32_t pos, float* hidden,
                                            uint32_t mode, void* stream) {
  // the step's workspace (the masked comparison path adds score rows for the
  // largest cache) must fit the library's buffer; other argument errors are
  // reported by sd_decode_step itself
  if (dims && layers && n_layers >= 1) {
    int max_cap = 0;
    if (mode & SD_ATTN_MASKED)
      for (int i = 0; i < n_layers; ++i)
        if (layers[i].cap_full > max_cap) max_cap = layers[i].cap_full;
    const size_t need = sd_workspace_bytes(dims, max_cap, 0);
    if (need > kScratchBytes) {
      char msg[200];
      snprintf(msg, sizeof msg,
               "sd_decode_step_noalloc: the step needs %zu bytes of scratch, above the "
               "library's %zu",
               need, kScratchBytes);
      return sd::set_error(SD_ENOSPC, msg);
    }
  }
  void* ws = nullptr;
  const sd_status st = scratch_of_current_device(&ws);
  if (st != SD_OK) return st;
  return sd_decode_step(dims, n_layers, layers, pos, hidden, mode, ws, kScratchBytes, stream);
}
