// Opt-in per-kernel timing: while on, every kernel launch of the library
// carries a start and a stop event that the dispatch itself records (kernel
// execution time); sd_profile_stop waits for them and reports, per kernel
// kind, the launch count and the summed time.  Off by default; the state is
// process-wide.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/sd.h"
#include "internal.hpp"

namespace sd {
namespace {

struct Rec {
  int kind;
  hipEvent_t a, b;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

const char* kKindNames[K_COUNT] = {
    "qkv_rope_append", "attn_partial",  "attn_combine",    "o_residual",    "cats_gate_up",
    "cats_down",       "cats_reduce", "sel_lse_partial", "sel_lse_final", "sel_score",
    "sel_topk",        "sel_gather",    "kth_select",      "masked_scores", "masked_softmax",
    "masked_pv",       "teal_qkv",      "teal_zero",       "teal_o",        "teal_gate_up",
    "teal_down",       "batch_qkv",     "batch_rope",      "batch_o",       "batch_gate_up",
    "batch_down",      "pack_tiles"};

}  // namespace

ProfEvents prof_events(int kind) {
  ProfEvents e;
  if (kind < 0) return e;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_on) return e;
  Rec r{kind, take_event(), take_event()};
  if (!r.a || !r.b) return e;
  g_recs.push_back(r);
  e.start = r.a;
  e.stop = r.b;
  return e;
}

}  // namespace sd

extern "C" sd_status sd_profile_start(void) {
  std::lock_guard<std::mutex> lock(sd::g_mu);
  sd::g_on = true;
  return SD_OK;
}

extern "C" int32_t sd_profile_stop(sd_kernel_stat* out, int32_t max_stats) {
  std::vector<sd::Rec> recs;
  {
    std::lock_guard<std::mutex> lock(sd::g_mu);
    sd::g_on = false;
    recs.swap(sd::g_recs);
  }
  int32_t launches[sd::K_COUNT] = {0};
  double ms[sd::K_COUNT] = {0};
  bool ok = true;
  for (auto& r : recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) ok = false;
    float t = 0.f;
    if (ok && hipEventElapsedTime(&t, r.a, r.b) == hipSuccess) {
      launches[r.kind] += 1;
      ms[r.kind] += t;
    }
  }
  {
    std::lock_guard<std::mutex> lock(sd::g_mu);
    for (auto& r : recs) {
      sd::g_pool.push_back(r.a);
      sd::g_pool.push_back(r.b);
    }
  }
  if (!ok) return -1;
  int32_t n = 0;
  for (int k = 0; k < sd::K_COUNT; ++k) {
    if (!launches[k]) continue;
    if (out && n < max_stats) {
      std::memset(out[n].name, 0, sizeof out[n].name);
      std::strncpy(out[n].name, sd::kKindNames[k], sizeof out[n].name - 1);
      out[n].launches = launches[k];
      out[n].total_ms = ms[k];
    }
    ++n;
  }
  return n;
}
