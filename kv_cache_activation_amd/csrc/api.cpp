// C ABI of the sparse decode-step library: argument checks, workspace layout
// and the order of kernel launches.  Every check runs before anything is
// enqueued, so a failing call leaves the stream untouched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/sd.h"
#include "internal.hpp"

namespace {

thread_local char g_err[512] = "";

sd_status fail(sd_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

bool aligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxSplits = 256;        // split-K chunks per KV head (the merge's capacity)
constexpr int kSplitBlocks = 256;      // auto mode: at most this many split workgroups
constexpr int kMinChunk = 64;          // auto mode: rows per split, lower bound
constexpr int kSelChunk = 256;         // key rows per selection workgroup
constexpr int kMaxWidth = 8192;        // widest GEMV input the kernels hold in VGPRs

size_t elem_size(int dtype) { return dtype == SD_BF16 ? 2 : 4; }

struct Layout {
  size_t q, attn, pm, pl, pacc, act, hmid, keep, mlp_part, teal_part, teal_tickets, lse_part,
      lse, scores;
  size_t teal_part_floats;
  size_t kth_hist, kth_state, topk, total;
  int max_splits, sel_chunks;
};

Layout make_layout(const sd_dims& dm, int max_rows, int max_window) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  const size_t hq = dm.n_q_heads, dh = dm.head_dim, hkv = dm.n_kv_heads, d = dm.d_model,
               ff = dm.d_ff;
  const size_t G = hq / hkv;
  L.max_splits = kMaxSplits;
  L.q = take(hq * dh * 4);
  L.attn = take(hq * dh * 4);
  L.pm = take(hq * L.max_splits * 4);
  L.pl = take(hq * L.max_splits * 4);
  L.pacc = take(hq * L.max_splits * dh * 4);
  L.act = take(ff * 4);
  L.hmid = take(ff * 4);
  L.keep = take(ff);
  L.mlp_part = take((size_t)sd::down_parts((int)ff) * d * 4);
  {  // TEAL partials: the largest of the layer's four sparse projections, at
     // the most slices any launch takes
    const int qkv_out = (int)((hq + 2 * hkv) * dh);
    auto need = [](int, int dout, int mats) {
      const size_t nblk = (dout + sd::kTealBlock - 1) / sd::kTealBlock;
      return (size_t)sd::kTealMaxSlices * nblk * sd::kTealBlock * mats;
    };
    size_t f = need((int)d, qkv_out, 1);
    f = std::max(f, need((int)(hq * dh), (int)d, 1));
    f = std::max(f, need((int)d, (int)ff, 2));
    f = std::max(f, need((int)ff, (int)d, 1));
    L.teal_part_floats = f;
    L.teal_part = take(f * 4);
    L.teal_tickets = take(sd::kTealMaxBlocks * 4);
  }
  L.sel_chunks = max_rows > 0 ? (max_rows + kSelChunk - 1) / kSelChunk : 0;
  L.lse_part = take(hkv * (size_t)L.sel_chunks * G * (size_t)max_window * 2 * 4);
  L.lse = take(hq * (size_t)max_window * 4);
  L.scores = take(hq * (size_t)max_rows * 4);  // masked comparison path: [h_q, rows]
  L.kth_hist = take(256 * 4);
  L.kth_state = take(16);
  L.topk = take(sd::topk_ws_words((int)hkv) * 4);
  L.total = off;
  return L;
}

sd_status check_dims(const sd_dims* dm) {
  if (!dm) return fail(SD_EINVAL, "dims is NULL");
  if (dm->d_model < 8 || dm->n_q_heads < 1 || dm->n_kv_heads < 1 || dm->d_ff < 1)
    return fail(SD_EINVAL, "dims must be positive");
  if (dm->n_q_heads % dm->n_kv_heads)
    return fail(SD_EINVAL, "n_q_heads %d is not a multiple of n_kv_heads %d", dm->n_q_heads,
                dm->n_kv_heads);
  const int G = dm->n_q_heads / dm->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(SD_EUNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8 (got %d)", G);
  if (dm->head_dim != 64 && dm->head_dim != 128)
    return fail(SD_EUNSUPPORTED, "head_dim must be 64 or 128 (got %d)", dm->head_dim);
  if (dm->d_model % 8 || dm->d_model > kMaxWidth)
    return fail(SD_EUNSUPPORTED, "d_model must be a multiple of 8 and at most %d", kMaxWidth);
  if (dm->n_q_heads * dm->head_dim > kMaxWidth)
    return fail(SD_EUNSUPPORTED, "n_q_heads * head_dim must be at most %d", kMaxWidth);
  if (dm->d_ff > sd::kDownList * sd::kDownMaxParts)
    return fail(SD_EUNSUPPORTED, "d_ff must be at most %d", sd::kDownList * sd::kDownMaxParts);
  if ((dm->w_dtype != SD_F32 && dm->w_dtype != SD_BF16) ||
      (dm->kv_dtype != SD_F32 && dm->kv_dtype != SD_BF16))
    return fail(SD_EUNSUPPORTED, "dtype must be SD_F32 or SD_BF16");
  if (!(dm->rms_eps >= 0.f)) return fail(SD_EINVAL, "rms_eps must be >= 0");
  return SD_OK;
}

sd_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SD_EHIP, "%s: %s", what, hipGetErrorString(e));
  return SD_OK;
}

int cu_count() {
  int dev = 0, cu = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev);
  return cu > 0 ? cu : 256;
}

// Split count of the split-K attention.  Measured on MI355X (partial +
// combine, bf16, 8 KV heads, caches rotated past the Infinity Cache): the
// launch costs about 9.5 us plus its bytes at 7.3 TB/s, and one workgroup per
// CU (kSplitBlocks = 256 chunks over all heads) is the fastest grid at every
// length from 3K to 128K rows per head (13114 rows: 16.8 us at 256 chunks,
// 17.9 at 512, 23.7 at 1024).  So: chunks of at least kMinChunk rows, about
// kSplitBlocks of them over all heads, then the largest split count whose
// chunks (ceil(n_max / s) rows, the size the launch uses) number at most
// kSplitBlocks, at most kMaxSplits.  Ragged lengths count each head's own
// chunks; a long head among short ones then gets many splits.
int plan_splits(const sd::HeadInts& lens, int h_kv, int n_max) {
  long long total = 0;
  for (int h = 0; h < h_kv; ++h) total += lens.v[h];
  long long chunk = (total + kSplitBlocks - 1) / kSplitBlocks;
  if (chunk < kMinChunk) chunk = kMinChunk;
  int s = (int)((n_max + chunk - 1) / chunk);
  if (s > kMaxSplits) s = kMaxSplits;
  for (; s > 1; --s) {
    const int c = (n_max + s - 1) / s;
    long long blocks = 0;
    for (int h = 0; h < h_kv; ++h) blocks += (lens.v[h] + c - 1) / c;
    if (blocks <= kSplitBlocks) break;
  }
  return s < 1 ? 1 : s;
}

int auto_splits(int n_ctx, int h_kv) {
  sd::HeadInts lens{};
  for (int h = 0; h < h_kv && h < sd::kMaxKvHeads; ++h) lens.v[h] = n_ctx;
  // more KV heads than the table holds: equal lengths, so scale the count
  if (h_kv > sd::kMaxKvHeads) {
    int s = kSplitBlocks / h_kv;
    const int by_rows = (n_ctx + kMinChunk - 1) / kMinChunk;
    if (s > by_rows) s = by_rows;
    return s < 1 ? 1 : s;
  }
  return plan_splits(lens, h_kv, n_ctx);
}

// Attention paths (the step's mode bits select them).
enum Path { P_SPLITK = 0, P_MASKED = 1, P_FUSED = 2 };

// Enqueue attention over logical rows 0..n_ctx-1 (row j read from physical
// row j + (j >= sink ? shift : 0)); ws must hold the layout's attention
// buffers (and, for the masked path, its score rows for `cap` rows).
void enqueue_attn(const sd_dims& dm, const Layout& L, char* ws, const float* q, const void* k,
                  const void* v, int cap, int n_ctx, int sink, int shift, float scale,
                  int n_splits, Path path, float* out, float* lse, hipStream_t s,
                  const sd::HeadInts* lens = nullptr) {
  sd::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.cap = cap;
  a.n_ctx = n_ctx;
  a.h_q = dm.n_q_heads;
  a.h_kv = dm.n_kv_heads;
  a.dh = dm.head_dim;
  a.sink = sink;
  a.shift = shift;
  a.scale = scale;
  a.pm = reinterpret_cast<float*>(ws + L.pm);
  a.pl = reinterpret_cast<float*>(ws + L.pl);
  a.pacc = reinterpret_cast<float*>(ws + L.pacc);
  a.out = out;
  a.lse = lse;
  if (lens) {  // ragged per-head lengths (split-K path); n_ctx is their maximum
    a.ragged = 1;
    a.lens = *lens;
  }
  if (path == P_MASKED) {
    sd::launch_attn_masked(a, reinterpret_cast<float*>(ws + L.scores), dm.kv_dtype, s);
    return;
  }
  a.per_query_head = path == P_FUSED;
  if (path == P_FUSED) n_splits = 1;  // one pass per query head, no split-K
  a.chunk = (n_ctx + n_splits - 1) / n_splits;
  a.n_splits = (n_ctx + a.chunk - 1) / a.chunk;
  sd::launch_attn(a, dm.kv_dtype, s);
}

// The CATS gate with the up rows of the kept channels: act, keep bytes, and
// hmid in the workspace (zero where dropped).
float* enqueue_gate(const sd_dims& dm, const Layout& L, char* ws, const float* x,
                    const float* norm, const void* wg, const void* wu, float t, int gate_in,
                    float* act, uint8_t* keep, hipStream_t s) {
  sd::GateArgs g{};
  g.x = x;
  g.norm = norm;
  g.eps = dm.rms_eps;
  g.w_gate = wg;
  g.w_up = wu;
  g.d = dm.d_model;
  g.dff = dm.d_ff;
  g.t = t;
  g.gate_in = gate_in;
  g.act = act;
  g.keep = keep;
  g.hmid = reinterpret_cast<float*>(ws + L.hmid);
  g.n_states = 1;
  sd::launch_gate(g, dm.w_dtype, s);
  return g.hmid;
}

void enqueue_mlp(const sd_dims& dm, const Layout& L, char* ws, const float* x, const float* norm,
                 const void* wg, const void* wu, const void* wd, float t, int gate_in, float* act,
                 uint8_t* keep, float* y, int accumulate, int32_t* idx, int32_t* n_kept,
                 hipStream_t s) {
  sd::GateArgs g{};
  g.x = x;
  g.norm = norm;
  g.eps = dm.rms_eps;
  g.w_gate = wg;
  g.w_up = wu;
  g.d = dm.d_model;
  g.dff = dm.d_ff;
  g.t = t;
  g.gate_in = gate_in;
  g.act = act;
  g.keep = keep;
  g.hmid = reinterpret_cast<float*>(ws + L.hmid);
  g.n_states = 1;
  sd::launch_gate(g, dm.w_dtype, s);

  sd::DownArgs dn{};
  dn.w_down_t = wd;
  dn.d = dm.d_model;
  dn.dff = dm.d_ff;
  dn.keep = keep;
  dn.hmid = g.hmid;
  dn.partials = reinterpret_cast<float*>(ws + L.mlp_part);
  dn.y = y;
  dn.accumulate = accumulate;
  dn.idx_out = idx;
  dn.n_kept_out = n_kept;
  sd::launch_down(dn, dm.w_dtype, s);
}

// One TEAL projection over column blocks, epilogue included (the layout's
// partials and tickets; the tickets must be zero, and the launch leaves them
// zero).
sd::TealArgs teal_args(int kind, const sd_dims& dm, const Layout& L, char* ws, const float* x,
                       int d_in, const float* norm, float t, const void* w0, const void* w1,
                       int d_out, int epi) {
  sd::TealArgs a{};
  a.kind = kind;
  a.x = x;
  a.d_in = d_in;
  a.norm = norm;
  a.eps = dm.rms_eps;
  a.t = t;
  a.w0 = w0;
  a.w1 = w1;
  a.d_out = d_out;
  a.part = reinterpret_cast<float*>(ws + L.teal_part);
  a.tickets = reinterpret_cast<unsigned*>(ws + L.teal_tickets);
  a.epi = epi;
  a.t_next = -1.f;
  return a;
}

}  // namespace

namespace sd {
sd_status set_error(sd_status st, const char* msg) { return fail(st, "%s", msg); }
}  // namespace sd

extern "C" {

const char* sd_status_string(sd_status st) {
  switch (st) {
    case SD_OK: return "ok";
    case SD_EINVAL: return "invalid argument";
    case SD_ENOSPC: return "insufficient workspace or capacity";
    case SD_EUNSUPPORTED: return "unsupported shape or dtype";
    case SD_EHIP: return "HIP error";
  }
  return "unknown status";
}

const char* sd_last_error(void) { return g_err; }

size_t sd_workspace_bytes(const sd_dims* dims, int32_t max_rows, int32_t max_window) {
  if (check_dims(dims) != SD_OK || max_rows < 0 || max_window < 0) return 0;
  return make_layout(*dims, max_rows, max_window).total;
}

sd_status sd_select_kv(const sd_dims* dims, const void* k_full, const void* v_full,
                       int32_t cap_full, int32_t n, const float* q_window, int32_t w,
                       int32_t n_sink, int32_t k_keep, float* scores, int32_t* idx, void* k_sel,
                       void* v_sel, int32_t cap_sel, uint32_t flags, void* ws, size_t ws_bytes,
                       void* stream) {
  sd_status st = check_dims(dims);
  if (st) return st;
  const bool scores_in = flags & SD_SCORES_IN;
  if (!aligned(k_full) || !aligned(v_full) || !aligned(scores) || !aligned(idx) ||
      !aligned(k_sel) || !aligned(v_sel) || (!scores_in && !aligned(q_window)) || !aligned(ws))
    return fail(SD_EINVAL, "null or misaligned pointer");
  if (n < 1 || n > cap_full) return fail(SD_EINVAL, "need 1 <= n <= cap_full");
  if (w < 1 || w > n) return fail(SD_EINVAL, "need 1 <= w <= n");
  if (n_sink < 0) return fail(SD_EINVAL, "n_sink must be >= 0");
  if (k_keep < n && k_keep < n_sink + w)
    return fail(SD_EINVAL, "k_keep %d < n_sink + w = %d", k_keep, n_sink + w);
  const int k_eff = k_keep < n ? k_keep : n;
  if (cap_sel < k_eff) return fail(SD_ENOSPC, "cap_sel %d < kept rows %d", cap_sel, k_eff);
  const Layout L = make_layout(*dims, n, w);
  if (ws_bytes < L.total) return fail(SD_ENOSPC, "workspace %zu < %zu bytes", ws_bytes, L.total);
  char* wsb = static_cast<char*>(ws);
  sd::SelectArgs a{};
  a.k = k_full;
  a.v = v_full;
  a.cap_full = cap_full;
  a.n = n;
  a.q_win = q_window;
  a.w = w;
  a.n_sink = n_sink;
  a.k_keep = k_keep;
  a.h_q = dims->n_q_heads;
  a.h_kv = dims->n_kv_heads;
  a.dh = dims->head_dim;
  a.scores = scores;
  a.idx = idx;
  a.k_sel = k_sel;
  a.v_sel = v_sel;
  a.cap_sel = cap_sel;
  a.n_chunks = L.sel_chunks;
  a.lse_part = reinterpret_cast<float*>(wsb + L.lse_part);
  a.lse = reinterpret_cast<float*>(wsb + L.lse);
  a.topk_ws = reinterpret_cast<unsigned*>(wsb + L.topk);
  a.skip_scoring = scores_in;
  sd::launch_select(a, dims->kv_dtype, static_cast<hipStream_t>(stream));
  return check_launch("sd_select_kv");
}

sd_status sd_decode_attn(const sd_dims* dims, const float* q, const void* k, const void* v,
                         int32_t cap, int32_t n_ctx, float scale, int32_t n_splits, float* out,
                         float* lse, void* ws, size_t ws_bytes, void* stream) {
  sd_status st = check_dims(dims);
  if (st) return st;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(out) || !aligned(ws) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return fail(SD_EINVAL, "null or misaligned pointer");
  if (n_ctx < 1 || n_ctx > cap) return fail(SD_EINVAL, "need 1 <= n_ctx <= cap");
  if (!std::isfinite(scale)) return fail(SD_EINVAL, "scale must be finite");
  const Layout L = make_layout(*dims, 0, 0);
  if (ws_bytes < L.total) return fail(SD_ENOSPC, "workspace %zu < %zu bytes", ws_bytes, L.total);
  if (n_splits < 0) return fail(SD_EINVAL, "n_splits must be >= 0");
  if (n_splits > L.max_splits)
    return fail(SD_ENOSPC, "n_splits %d above the workspace's %d", n_splits, L.max_splits);
  int s = n_splits ? (n_splits < n_ctx ? n_splits : n_ctx) : auto_splits(n_ctx, dims->n_kv_heads);
  enqueue_attn(*dims, L, static_cast<char*>(ws), q, k, v, cap, n_ctx, n_ctx, 0, scale, s,
               P_SPLITK, out, lse, static_cast<hipStream_t>(stream));
  return check_launch("sd_decode_attn");
}

sd_status sd_select_kv_ragged(const sd_dims* dims, const void* k_full, const void* v_full,
                              int32_t cap_full, int32_t n, const float* q_window, int32_t w,
                              int32_t n_sink, const int32_t* k_keep_heads, float* scores,
                              int32_t* idx, int32_t idx_stride, void* k_sel, void* v_sel,
                              int32_t cap_sel, uint32_t flags, void* ws, size_t ws_bytes,
                              void* stream) {
  sd_status st = check_dims(dims);
  if (st) return st;
  const bool scores_in = flags & SD_SCORES_IN;
  if (!aligned(k_full) || !aligned(v_full) || !aligned(scores) || !aligned(idx) ||
      !aligned(k_sel) || !aligned(v_sel) || (!scores_in && !aligned(q_window)) || !aligned(ws) ||
      !k_keep_heads)
    return fail(SD_EINVAL, "null or misaligned pointer");
  if (dims->n_kv_heads > sd::kMaxKvHeads)
    return fail(SD_EUNSUPPORTED, "ragged budgets need n_kv_heads <= %d", sd::kMaxKvHeads);
  if (n < 1 || n > cap_full) return fail(SD_EINVAL, "need 1 <= n <= cap_full");
  if (w < 1 || w > n) return fail(SD_EINVAL, "need 1 <= w <= n");
  if (n_sink < 0) return fail(SD_EINVAL, "n_sink must be >= 0");
  sd::HeadInts kh{};
  int k_max = 0;
  for (int h = 0; h < dims->n_kv_heads; ++h) {
    const int k = k_keep_heads[h];
    if (k < n && k < n_sink + w)
      return fail(SD_EINVAL, "head %d: k_keep %d < n_sink + w = %d", h, k, n_sink + w);
    kh.v[h] = k;
    const int ke = k < n ? k : n;
    if (ke > k_max) k_max = ke;
  }
  if (idx_stride < k_max) return fail(SD_EINVAL, "idx_stride %d < largest kept count %d", idx_stride, k_max);
  if (cap_sel < k_max) return fail(SD_ENOSPC, "cap_sel %d < kept rows %d", cap_sel, k_max);
  const Layout L = make_layout(*dims, n, w);
  if (ws_bytes < L.total) return fail(SD_ENOSPC, "workspace %zu < %zu bytes", ws_bytes, L.total);
  char* wsb = static_cast<char*>(ws);
  sd::SelectArgs a{};
  a.k = k_full;
  a.v = v_full;
  a.cap_full = cap_full;
  a.n = n;
  a.q_win = q_window;
  a.w = w;
  a.n_sink = n_sink;
  a.k_keep = k_max;
  a.h_q = dims->n_q_heads;
  a.h_kv = dims->n_kv_heads;
  a.dh = dims->head_dim;
  a.scores = scores;
  a.idx = idx;
  a.k_sel = k_sel;
  a.v_sel = v_sel;
  a.cap_sel = cap_sel;
  a.n_chunks = L.sel_chunks;
  a.lse_part = reinterpret_cast<float*>(wsb + L.lse_part);
  a.lse = reinterpret_cast<float*>(wsb + L.lse);
  a.topk_ws = reinterpret_cast<unsigned*>(wsb + L.topk);
  a.skip_scoring = scores_in;
  a.ragged = 1;
  a.k_heads = kh;
  a.idx_stride = idx_stride;
  sd::launch_select(a, dims->kv_dtype, static_cast<hipStream_t>(stream));
  return check_launch("sd_select_kv_ragged");
}

sd_status sd_decode_attn_ragged(const sd_dims* dims, const float* q, const void* k, const void* v,
                                int32_t cap, const int32_t* n_ctx_heads, float scale,
                                int32_t n_splits, float* out, float* lse, void* ws,
                                size_t ws_bytes, void* stream) {
  sd_status st = check_dims(dims);
  if (st) return st;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(out) || !aligned(ws) ||
      !n_ctx_heads || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return fail(SD_EINVAL, "null or misaligned pointer");
  if (dims->n_kv_heads > sd::kMaxKvHeads)
    return fail(SD_EUNSUPPORTED, "ragged lengths need n_kv_heads <= %d", sd::kMaxKvHeads);
  sd::HeadInts lens{};
  int n_max = 0;
  for (int h = 0; h < dims->n_kv_heads; ++h) {
    if (n_ctx_heads[h] < 1 || n_ctx_heads[h] > cap)
      return fail(SD_EINVAL, "head %d: need 1 <= n_ctx <= cap", h);
    lens.v[h] = n_ctx_heads[h];
    if (lens.v[h] > n_max) n_max = lens.v[h];
  }
  if (!std::isfinite(scale)) return fail(SD_EINVAL, "scale must be finite");
  const Layout L = make_layout(*dims, 0, 0);
  if (ws_bytes < L.total) return fail(SD_ENOSPC, "workspace %zu < %zu bytes", ws_bytes, L.total);
  if (n_splits < 0) return fail(SD_EINVAL, "n_splits must be >= 0");
  if (n_splits > L.max_splits)
    return fail(SD_ENOSPC, "n_splits %d above the workspace's %d", n_splits, L.max_splits);
  int sp = n_splits ? (n_splits < n_max ? n_splits : n_max)
                    : plan_splits(lens, dims->n_kv_heads, n_max);
  enqueue_attn(*dims, L, static_cast<char*>(ws), q, k, v, cap, n_max, n_max, 0, scale, sp,
               P_SPLITK, out, lse, static_cast<hipStream_t>(stream), &lens);
  return check_launch("sd_decode_attn_ragged");
}

sd_status sd_decode_attn_window(const sd_dims* dims, const float* q, const void* k, const void* v,
                                int32_t cap, int32_t n_rows, int32_t n_sink, int32_t n_keep,
                                float scale, int32_t n_splits, float* out, float* lse, void* ws,
                                size_t ws_bytes, void* stream) {
  sd_status st = check_dims(dims);
  if (st) return st;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(out) || !aligned(ws) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return fail(SD_EINVAL, "null or misaligned pointer");
  if (n_rows < 1 || n_rows > cap) return fail(SD_EINVAL, "need 1 <= n_rows <= cap");
  if (n_keep < 1 || n_sink < 0 || n_sink > n_keep)
    return fail(SD_EINVAL, "need 0 <= n_sink <= n_keep and n_keep >= 1");
  if (!std::isfinite(scale)) return fail(SD_EINVAL, "scale must be finite");
  const Layout L = make_layout(*dims, 0, 0);
  if (ws_bytes < L.total) return fail(SD_ENOSPC, "workspace %zu < %zu bytes", ws_bytes, L.total);
  if (n_splits < 0) return fail(SD_EINVAL, "n_splits must be >= 0");
  if (n_splits > L.max_splits)
    return fail(SD_ENOSPC, "n_splits %d above the workspace's %d", n_splits, L.max_splits);
  const int n_ctx = n_keep < n_rows ? n_keep : n_rows;
  const int sink = n_keep < n_rows ? n_sink : n_ctx;
  const int shift = n_keep < n_rows ? n_rows - n_keep : 0;
  int s = n_splits ? (n_splits < n_ctx ? n_splits : n_ctx) : auto_splits(n_ctx, dims->n_kv_heads);
  enqueue_attn(*dims, L, static_cast<char*>(ws), q, k, v, cap, n_ctx, sink, shift, scale, s,
               P_SPLITK, out, lse, static_cast<hipStream_t>(stream));
  return check_launch("sd_decode_attn_window");
}

sd_status sd_decode_attn_baseline(const sd_dims* dims, const float* q, const void* k,
                                  const void* v, int32_t cap, int32_t n_ctx, float scale,
                                  int32_t path, float* out, float* lse, void* ws, size_t ws_bytes,
                                  void* stream) {
  sd_status st = check_dims(dims);
  if (st) return st;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(out) || !aligned(ws) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return fail(SD_EINVAL, "null or misaligned pointer");
  if (n_ctx < 1 || n_ctx > cap) return fail(SD_EINVAL, "need 1 <= n_ctx <= cap");
  if (!std::isfinite(scale)) return fail(SD_EINVAL, "scale must be finite");
  if (path != SD_ATTN_MASKED && path != SD_ATTN_FUSED)
    return fail(SD_EINVAL, "path must be SD_ATTN_MASKED or SD_ATTN_FUSED");
  const Layout L = make_layout(*dims, path == SD_ATTN_MASKED ? cap : 0, 0);
  if (ws_bytes < L.total) return fail(SD_ENOSPC, "workspace %zu < %zu bytes", ws_bytes, L.total);
  enqueue_attn(*dims, L, static_cast<char*>(ws), q, k, v, cap, n_ctx, n_ctx, 0, scale, 1,
               path == SD_ATTN_MASKED ? P_MASKED : P_FUSED, out, lse,
               static_cast<hipStream_t>(stream));
  return check_launch("sd_decode_attn_baseline");
}

sd_status sd_sparse_mlp(const sd_dims* dims, const float* x, const float* norm_w,
                        const void* w_gate, const void* w_up, const void* w_down_t,
                        float threshold, float* y, float* act, int32_t* idx, int32_t* n_kept,
                        uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  sd_status st = check_dims(dims);
  if (st) return st;
  const bool gate_in = flags & SD_GATE_IN;
  if (!aligned(x) || (norm_w && !aligned(norm_w)) || (!gate_in && !aligned(w_gate)) ||
      !aligned(w_up) || !aligned(w_down_t) || !aligned(y) || !aligned(act) || !aligned(idx) ||
      !n_kept || !aligned(ws))
    return fail(SD_EINVAL, "null or misaligned pointer");
  if (std::isnan(threshold)) return fail(SD_EINVAL, "threshold is NaN");
  const Layout L = make_layout(*dims, 0, 0);
  if (ws_bytes < L.total) return fail(SD_ENOSPC, "workspace %zu < %zu bytes", ws_bytes, L.total);
  char* wsb = static_cast<char*>(ws);
  enqueue_mlp(*dims, L, wsb, x, norm_w, w_gate, w_up, w_down_t, threshold, gate_in, act,
              reinterpret_cast<uint8_t*>(wsb + L.keep), y, 0, idx, n_kept,
              static_cast<hipStream_t>(stream));
  return check_launch("sd_sparse_mlp");
}

sd_status sd_teal_gemv(const sd_dims* dims, const float* x, int32_t d_in, const float* norm_w,
                       float threshold, const void* w_t, const void* w2_t, int32_t d_out,
                       float* y, float* y2, uint32_t flags, int32_t* idx, int32_t* n_kept,
                       void* ws, size_t ws_bytes, void* stream) {
  sd_status st = check_dims(dims);
  if (st) return st;
  if (!aligned(x) || (norm_w && !aligned(norm_w)) || !aligned(w_t) || !aligned(y) ||
      !aligned(ws) || (idx && !aligned(idx)) || (w2_t && (!aligned(w2_t) || !aligned(y2))))
    return fail(SD_EINVAL, "null or misaligned pointer");
  if (flags & ~(uint32_t)SD_ACCUMULATE) return fail(SD_EINVAL, "unknown flags 0x%x", flags);
  if (d_in < 8 || d_out < 8 || d_in % 8 || d_out % 8)
    return fail(SD_EINVAL, "d_in and d_out must be positive multiples of 8");
  if (d_in > 32768) return fail(SD_EUNSUPPORTED, "d_in must be at most 32768");
  if (std::isnan(threshold)) return fail(SD_EINVAL, "threshold is NaN");
  const Layout L = make_layout(*dims, 0, 0);
  if (ws_bytes < L.total) return fail(SD_ENOSPC, "workspace %zu < %zu bytes", ws_bytes, L.total);
  const int nblk = (d_out + sd::kTealBlock - 1) / sd::kTealBlock;
  const int mats = w2_t ? 2 : 1;
  const size_t need = (size_t)sd::teal_slices(d_in, d_out) * nblk * sd::kTealBlock * mats;
  if (need > L.teal_part_floats || nblk > sd::kTealMaxBlocks)
    return fail(SD_ENOSPC, "d_in %d x d_out %d needs %zu partial floats, the workspace holds %zu",
                d_in, d_out, need, L.teal_part_floats);
  char* wsb = static_cast<char*>(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  sd::TealArgs a = teal_args(sd::K_TEAL_O, *dims, L, wsb, x, d_in, norm_w, threshold, w_t, w2_t,
                             d_out, (flags & SD_ACCUMULATE) ? sd::TEAL_ACC : sd::TEAL_STORE);
  a.y = y;
  a.y2 = y2;
  a.idx_out = idx;
  a.n_kept_out = n_kept;
  sd::launch_teal_zero(a.tickets, nblk, s);
  sd::launch_teal(a, dims->w_dtype, dims->kv_dtype, s);
  return check_launch("sd_teal_gemv");
}

sd_status sd_stream_read(const void* buf, size_t bytes, uint32_t* out, void* stream) {
  if (!aligned(buf) || !aligned(out)) return fail(SD_EINVAL, "null or misaligned pointer");
  if (bytes == 0 || bytes % 8192)
    return fail(SD_EINVAL, "bytes must be a positive multiple of 8192 (got %zu)", bytes);
  sd::launch_stream_read(buf, bytes, out, static_cast<hipStream_t>(stream));
  return check_launch("sd_stream_read");
}

sd_status sd_pack_tiles(const void* w, int32_t rows, int32_t d_in, void* out, void* stream) {
  if (!aligned(w) || !aligned(out)) return fail(SD_EINVAL, "null or misaligned pointer");
  if (rows < 1 || d_in < 8 || d_in % 8)
    return fail(SD_EINVAL, "rows must be positive and d_in a positive multiple of 8");
  const size_t in_bytes = (size_t)rows * d_in * 2, out_bytes = SD_TILE_BYTES(rows, d_in);
  const uintptr_t a = reinterpret_cast<uintptr_t>(w), b = reinterpret_cast<uintptr_t>(out);
  if (a < b + out_bytes && b < a + in_bytes) return fail(SD_EINVAL, "out overlaps w");
  sd::launch_pack_tiles(w, rows, d_in, out, static_cast<hipStream_t>(stream));
  return check_launch("sd_pack_tiles");
}

sd_status sd_decode_step(const sd_dims* dims, int32_t n_layers, sd_layer* layers, int32_t pos,
                         float* hidden, uint32_t mode, void* ws, size_t ws_bytes, void* stream) {
  sd_status st = check_dims(dims);
  if (st) return st;
  if (n_layers < 1 || !layers) return fail(SD_EINVAL, "need n_layers >= 1 and a layer array");
  if (!aligned(hidden) || !aligned(ws)) return fail(SD_EINVAL, "null or misaligned pointer");
  if (pos < 0) return fail(SD_EINVAL, "pos must be >= 0");
  const bool kv_sparse = mode & SD_KV_SPARSE, mlp_sparse = mode & SD_MLP_SPARSE;
  const bool kv_window = mode & SD_KV_WINDOW;
  const bool masked = mode & SD_ATTN_MASKED, fused = mode & SD_ATTN_FUSED;
  const bool teal = mode & SD_PROJ_TEAL;
  if (mode & ~(uint32_t)(SD_KV_SPARSE | SD_MLP_SPARSE | SD_KV_WINDOW | SD_ATTN_MASKED |
                         SD_ATTN_FUSED | SD_PROJ_TEAL))
    return fail(SD_EINVAL, "unknown mode bits 0x%x", mode);
  if (teal && mlp_sparse) return fail(SD_EINVAL, "SD_PROJ_TEAL excludes SD_MLP_SPARSE");
  if ((int)kv_sparse + (int)kv_window + (int)masked + (int)fused > 1)
    return fail(SD_EINVAL, "at most one of SD_KV_SPARSE, SD_KV_WINDOW, SD_ATTN_MASKED, SD_ATTN_FUSED");
  int max_cap = 0;
  for (int i = 0; i < n_layers; ++i)
    if (layers[i].cap_full > max_cap) max_cap = layers[i].cap_full;
  const Layout L = make_layout(*dims, masked ? max_cap : 0, 0);
  if (ws_bytes < L.total) return fail(SD_ENOSPC, "workspace %zu < %zu bytes", ws_bytes, L.total);
  bool blk_down = false;  // some layer's down projection reads column blocks
  for (int i = 0; i < n_layers; ++i) blk_down = blk_down || layers[i].w_down_b != nullptr;
  if (blk_down && (dims->d_model + sd::kTealBlock - 1) / sd::kTealBlock > sd::kTealMaxBlocks)
    return fail(SD_EUNSUPPORTED, "w_down_b: d_model above %d", sd::kTealMaxBlocks * sd::kTealBlock);
  for (int i = 0; i < n_layers; ++i) {
    const sd_layer& l = layers[i];
    if (!aligned(l.attn_norm) || !aligned(l.mlp_norm) || !aligned(l.w_down_t) ||
        !aligned(l.k_full) || !aligned(l.v_full))
      return fail(SD_EINVAL, "layer %d: null or misaligned pointer", i);
    if (teal) {
      if (!aligned(l.w_qkv_t) || !aligned(l.w_o_t) || !aligned(l.w_gate_t) || !aligned(l.w_up_t))
        return fail(SD_EINVAL, "layer %d: SD_PROJ_TEAL needs the column-block weights", i);
      for (int k = 0; k < 4; ++k)
        if (std::isnan(l.teal_t[k])) return fail(SD_EINVAL, "layer %d: TEAL threshold is NaN", i);
      if (l.teal_masks_out && !aligned(l.teal_masks_out))
        return fail(SD_EINVAL, "layer %d: misaligned teal_masks_out", i);
    } else if (!aligned(l.w_qkv) || !aligned(l.w_o) || !aligned(l.w_gate) || !aligned(l.w_up)) {
      return fail(SD_EINVAL, "layer %d: null or misaligned pointer", i);
    }
    if (l.n_full < 0 || l.n_full >= l.cap_full)
      return fail(SD_ENOSPC, "layer %d: full cache has no free row (n_full %d, cap %d)", i,
                  l.n_full, l.cap_full);
    if (l.k_sel || l.v_sel) {
      if (!aligned(l.k_sel) || !aligned(l.v_sel))
        return fail(SD_EINVAL, "layer %d: misaligned gathered buffer", i);
      if (l.n_sel_heads) {
        if (dims->n_kv_heads > sd::kMaxKvHeads)
          return fail(SD_EUNSUPPORTED, "ragged budgets need n_kv_heads <= %d", sd::kMaxKvHeads);
        if (kv_window) return fail(SD_EINVAL, "layer %d: ragged budgets exclude the window", i);
        for (int h = 0; h < dims->n_kv_heads; ++h)
          if (l.n_sel_heads[h] < 0 || l.n_sel_heads[h] >= l.cap_sel)
            return fail(SD_ENOSPC, "layer %d head %d: gathered buffer has no free row", i, h);
      } else if (l.n_sel < 0 || l.n_sel >= l.cap_sel) {
        return fail(SD_ENOSPC, "layer %d: gathered buffer has no free row (n_sel %d, cap %d)",
                    i, l.n_sel, l.cap_sel);
      }
    } else if (kv_sparse) {
      return fail(SD_EINVAL, "layer %d: KV-sparse mode needs a gathered buffer", i);
    }
    if (std::isnan(l.cats_threshold)) return fail(SD_EINVAL, "layer %d: threshold is NaN", i);
    if (l.mask_out && !aligned(l.mask_out))
      return fail(SD_EINVAL, "layer %d: misaligned mask_out", i);
    if (l.w_down_b && !aligned(l.w_down_b))
      return fail(SD_EINVAL, "layer %d: misaligned w_down_b", i);
    if (kv_window && (l.window_keep < 1 || l.window_sink < 0 || l.window_sink > l.window_keep))
      return fail(SD_EINVAL, "layer %d: need 0 <= window_sink <= window_keep, window_keep >= 1", i);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* wsb = static_cast<char*>(ws);
  float* q = reinterpret_cast<float*>(wsb + L.q);
  float* attn = reinterpret_cast<float*>(wsb + L.attn);
  const int d = dims->d_model, hq = dims->n_q_heads, dh = dims->head_dim, hkv = dims->n_kv_heads;
  const float scale = 1.0f / std::sqrt((float)dh);
  // RoPE angles pos * theta^(-2i/d_h) in double precision (theta <= 0: identity)
  sd::RopeTable rope{};
  for (int i = 0; i < dh / 2; ++i) {
    rope.c[i] = 1.0f;
    rope.s[i] = 0.0f;
    if (dims->rope_theta > 0.f) {
      const double ang = (double)pos * std::pow((double)dims->rope_theta, -2.0 * i / (double)dh);
      rope.c[i] = (float)std::cos(ang);
      rope.s[i] = (float)std::sin(ang);
    }
  }
  for (int i = 0; i < n_layers; ++i) {
    const sd_layer& l = layers[i];
    const bool has_sel = l.k_sel != nullptr;
    sd::QkvArgs qa{};
    qa.h = hidden;
    qa.norm = l.attn_norm;
    qa.eps = dims->rms_eps;
    qa.w = l.w_qkv;
    qa.d = d;
    qa.h_q = hq;
    qa.h_kv = hkv;
    qa.dh = dh;
    qa.rope = rope;
    qa.q_out = q;
    qa.k_full = l.k_full;
    qa.v_full = l.v_full;
    qa.cap_full = l.cap_full;
    qa.row_full = l.n_full;
    qa.k_sel = has_sel ? l.k_sel : nullptr;
    qa.v_sel = has_sel ? l.v_sel : nullptr;
    qa.cap_sel = l.cap_sel;
    qa.row_sel = l.n_sel;
    sd::HeadInts lens{};  // ragged budgets: per-head append rows, then per-head lengths
    int n_ragged = 0;
    if (has_sel && l.n_sel_heads) {
      qa.ragged = 1;
      for (int h = 0; h < hkv; ++h) {
        qa.sel_rows.v[h] = l.n_sel_heads[h];
        lens.v[h] = l.n_sel_heads[h] + 1;
        if (lens.v[h] > n_ragged) n_ragged = lens.v[h];
      }
    }
    const int qkv_out = (hq + 2 * hkv) * dh;
    uint8_t* tm = teal ? l.teal_masks_out : nullptr;  // [d | h_q d_h | d | d_ff]
    if (i == 0 && (teal || blk_down))  // every column-block launch leaves its tickets zero
      sd::launch_teal_zero(reinterpret_cast<unsigned*>(wsb + L.teal_tickets), sd::kTealMaxBlocks,
                           s);
    if (teal) {
      sd::TealArgs a = teal_args(sd::K_TEAL_QKV, *dims, L, wsb, hidden, d, l.attn_norm,
                                 l.teal_t[0], l.w_qkv_t, nullptr, qkv_out, sd::TEAL_QKV);
      a.qkv = qa;
      a.keep_out = tm;
      sd::launch_teal(a, dims->w_dtype, dims->kv_dtype, s);
    } else {
      sd::launch_qkv(qa, dims->w_dtype, dims->kv_dtype, s);
    }

    const void* kc = kv_sparse ? l.k_sel : l.k_full;
    const void* vc = kv_sparse ? l.v_sel : l.v_full;
    const int cap = kv_sparse ? l.cap_sel : l.cap_full;
    int n_ctx = (kv_sparse ? l.n_sel : l.n_full) + 1;
    int sink = n_ctx, shift = 0;
    if (kv_window && l.window_keep < n_ctx) {  // sinks + most recent rows, in place
      shift = n_ctx - l.window_keep;
      sink = l.window_sink;
      n_ctx = l.window_keep;
    }
    const Path path = masked ? P_MASKED : fused ? P_FUSED : P_SPLITK;
    const bool ragged = kv_sparse && qa.ragged;
    if (ragged) n_ctx = sink = n_ragged;
    const int splits = ragged ? plan_splits(lens, hkv, n_ctx) : auto_splits(n_ctx, hkv);
    enqueue_attn(*dims, L, wsb, q, kc, vc, cap, n_ctx, sink, shift, scale, splits, path, attn,
                 nullptr, s, ragged ? &lens : nullptr);

    if (teal) {
      float* hmid = reinterpret_cast<float*>(wsb + L.hmid);
      const int ff = dims->d_ff;
      // O: attention output -> h += W_o (mask * attn)
      sd::TealArgs ao = teal_args(sd::K_TEAL_O, *dims, L, wsb, attn, hq * dh, nullptr,
                                  l.teal_t[1], l.w_o_t, nullptr, d, sd::TEAL_ACC);
      ao.y = hidden;
      ao.keep_out = tm ? tm + d : nullptr;
      sd::launch_teal(ao, dims->w_dtype, dims->kv_dtype, s);
      // gate and up share the MLP input; hmid = SiLU(gate) * up.  The epilogue
      // also decides the down projection's input mask: without w_down_b the
      // down projection is the kept-row kernel of the CATS branch (w_down_t is
      // the same [d_ff, d] layout), which ranks those keep bytes instead of
      // re-reading and re-testing the float input in every workgroup
      uint8_t* dkeep = tm ? tm + 2 * d + hq * dh : reinterpret_cast<uint8_t*>(wsb + L.keep);
      sd::TealArgs ag = teal_args(sd::K_TEAL_GATE_UP, *dims, L, wsb, hidden, d, l.mlp_norm,
                                  l.teal_t[2], l.w_gate_t, l.w_up_t, ff, sd::TEAL_SWIGLU);
      ag.y = hmid;
      ag.t_next = l.teal_t[3];
      ag.keep_next = dkeep;
      ag.keep_out = tm ? tm + d + hq * dh : nullptr;
      sd::launch_teal(ag, dims->w_dtype, dims->kv_dtype, s);
      if (l.w_down_b) {  // down over column blocks: |hmid| > t tested per slice again
        sd::TealArgs db = teal_args(sd::K_TEAL_DOWN, *dims, L, wsb, hmid, ff, nullptr, l.teal_t[3],
                                    l.w_down_b, nullptr, d, sd::TEAL_DOWN);
        db.y = hidden;
        sd::launch_teal(db, dims->w_dtype, dims->kv_dtype, s);
        continue;
      }
      // down: h += W_down (mask * hmid)
      sd::DownArgs dn{};
      dn.w_down_t = l.w_down_t;
      dn.d = d;
      dn.dff = ff;
      dn.keep = dkeep;
      dn.hmid = hmid;
      dn.partials = reinterpret_cast<float*>(wsb + L.mlp_part);
      dn.y = hidden;
      dn.accumulate = 1;
      sd::launch_down(dn, dims->w_dtype, s);
      continue;
    }
    sd::launch_o(attn, l.w_o, hq * dh, d, hidden, dims->w_dtype, s);

    uint8_t* keep = l.mask_out ? l.mask_out : reinterpret_cast<uint8_t*>(wsb + L.keep);
    const float t_mlp = mlp_sparse ? l.cats_threshold : -1.0f;
    if (l.w_down_b) {
      // the gate writes hmid, zero where a channel is dropped; the down
      // projection over column blocks then reads the pieces of the channels
      // with hmid != 0 (dense: every channel), partial sums inside the launch
      float* hm = enqueue_gate(*dims, L, wsb, hidden, l.mlp_norm, l.w_gate, l.w_up, t_mlp, 0,
                               reinterpret_cast<float*>(wsb + L.act), keep, s);
      sd::TealArgs db = teal_args(sd::K_DOWN, *dims, L, wsb, hm, dims->d_ff, nullptr,
                                  mlp_sparse ? 0.0f : -1.0f, l.w_down_b, nullptr, d,
                                  sd::TEAL_CATS_DOWN);
      db.y = hidden;
      sd::launch_teal(db, dims->w_dtype, dims->kv_dtype, s);
      continue;
    }
    enqueue_mlp(*dims, L, wsb, hidden, l.mlp_norm, l.w_gate, l.w_up, l.w_down_t, t_mlp, 0,
                reinterpret_cast<float*>(wsb + L.act), keep, hidden, 1, nullptr, nullptr, s);
  }
  st = check_launch("sd_decode_step");
  if (st) return st;
  for (int i = 0; i < n_layers; ++i) {
    layers[i].n_full += 1;
    if (layers[i].k_sel) {
      if (layers[i].n_sel_heads) {
        for (int h = 0; h < dims->n_kv_heads; ++h) layers[i].n_sel_heads[h] += 1;
      } else {
        layers[i].n_sel += 1;
      }
    }
  }
  return SD_OK;
}

// Batched decode: the single-sequence layout (attention partials, reused by
// every sequence in stream order) plus the batch's own buffers.
struct BatchLayout {
  Layout base;
  size_t qkv, q, attn, pm, pl, pacc, act, hmid, keep, uni, part, mm_part, mm_ssq, mm_tickets,
      rope, total;
  int mm_groups;
};

BatchLayout make_batch_layout(const sd_dims& dm, int nb) {
  BatchLayout B{};
  B.base = make_layout(dm, 0, 0);
  size_t off = B.base.total;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  const size_t hq = dm.n_q_heads, dh = dm.head_dim, hkv = dm.n_kv_heads, d = dm.d_model,
               ff = dm.d_ff, n = nb;
  B.qkv = take(n * (hq + 2 * hkv) * dh * 4);
  B.q = take(n * hq * dh * 4);
  B.attn = take(n * hq * dh * 4);
  B.pm = take(n * hq * kMaxSplits * 4);
  B.pl = take(n * hq * kMaxSplits * 4);
  B.pacc = take(n * hq * kMaxSplits * dh * 4);
  B.act = take(n * ff * 4);
  B.hmid = take(n * ff * 4);
  B.keep = take(n * ff);
  B.uni = take(ff);
  B.part = take((size_t)sd::down_parts((int)ff) * n * d * 4);
  B.rope = take(n * (dh / 2) * 2 * 4);
  {  // matrix-core path: the largest of the layer's four launches
    const int qo = (int)((hq + 2 * hkv) * dh), od = (int)(hq * dh);
    const size_t pf = std::max(std::max(sd::bmma_part_floats(qo, (int)d, false),
                                        sd::bmma_part_floats((int)d, od, false)),
                               std::max(sd::bmma_part_floats((int)ff, (int)d, true),
                                        sd::bmma_part_floats((int)d, (int)ff, false)));
    const size_t sf = std::max(sd::bmma_ssq_floats(qo, (int)d, false),
                               sd::bmma_ssq_floats((int)ff, (int)d, true));
    const int groups = std::max(std::max(sd::bmma_groups(qo), sd::bmma_groups((int)d)),
                                sd::bmma_groups((int)ff));
    B.mm_part = take(pf * 4);
    B.mm_ssq = take(sf * 4);
    B.mm_tickets = take((size_t)groups * 4);
    B.mm_groups = groups;
  }
  B.total = off;
  return B;
}

// Chunks of the batched attention: one chunk size c for every sequence, about
// kSplitBlocks chunk workgroups over all (sequence, KV head) pairs and never
// more (the measured cliff of the split-K kernel), at least kMinChunk rows,
// at most kMaxSplits chunks per head; then each sequence's chunk is evened
// out over its split count.
void plan_batch_splits(const int* rows, int nb, int hkv, long long total, sd::AttnBatch& bt) {
  long long c = (total + kSplitBlocks - 1) / kSplitBlocks;
  if (c < kMinChunk) c = kMinChunk;
  for (;;) {
    long long blocks = 0, most = 1;
    for (int b = 0; b < nb; ++b) {
      long long sp = (rows[b] + c - 1) / c;
      if (sp > kMaxSplits) sp = kMaxSplits;
      if (sp > most) most = sp;
      blocks += hkv * sp;
    }
    // stop at the cap, or once every sequence is down to one chunk per head
    // (more (sequence, KV head) pairs than the cap: one chunk each, as many
    // workgroups as pairs)
    if (blocks <= kSplitBlocks || most == 1) break;
    c += c / 16 + 1;
  }
  int start = 0;
  for (int b = 0; b < 8; ++b) {
    if (b >= nb) {
      bt.starts[b] = INT_MAX;
      continue;
    }
    int sp = (int)((rows[b] + c - 1) / c);
    if (sp > kMaxSplits) sp = kMaxSplits;
    if (sp < 1) sp = 1;
    bt.chunk[b] = (rows[b] + sp - 1) / sp;
    bt.splits[b] = (rows[b] + bt.chunk[b] - 1) / bt.chunk[b];
    bt.starts[b] = start;
    start += hkv * bt.splits[b];
  }
}

sd_status check_batch_dims(const sd_dims* dims, int32_t batch) {
  sd_status st = check_dims(dims);
  if (st) return st;
  if (batch < 2 || batch > sd::kMaxBatch)
    return fail(SD_EINVAL, "batch must be 2..%d (one sequence: sd_decode_step)", sd::kMaxBatch);
  if (dims->d_model > 4096 || dims->n_q_heads * dims->head_dim > 4096)
    return fail(SD_EUNSUPPORTED, "batched step: d_model and n_q_heads * head_dim at most 4096");
  return SD_OK;
}

size_t sd_batch_workspace_bytes(const sd_dims* dims, int32_t batch) {
  if (check_batch_dims(dims, batch) != SD_OK) return 0;
  return make_batch_layout(*dims, batch).total;
}

sd_status sd_decode_step_batch(const sd_dims* dims, int32_t n_layers, const sd_layer* layers,
                               int32_t batch, sd_seq_kv* kv, const int32_t* pos, float* hidden,
                               uint32_t mode, void* ws, size_t ws_bytes, void* stream) {
  sd_status st = check_batch_dims(dims, batch);
  if (st) return st;
  if (n_layers < 1 || !layers || !kv || !pos || !aligned(hidden) || !aligned(ws))
    return fail(SD_EINVAL, "null or misaligned argument");
  if (mode & ~(uint32_t)(SD_KV_SPARSE | SD_MLP_SPARSE | SD_MATRIX_CORES))
    return fail(SD_EINVAL,
                "batched step modes: SD_KV_SPARSE and/or SD_MLP_SPARSE, optionally SD_MATRIX_CORES");
  const bool kv_sparse = mode & SD_KV_SPARSE, mlp_sparse = mode & SD_MLP_SPARSE;
  const bool mc = mode & SD_MATRIX_CORES;
  if (mc && dims->w_dtype != SD_BF16)
    return fail(SD_EUNSUPPORTED, "SD_MATRIX_CORES needs bf16 weights");
  const BatchLayout B = make_batch_layout(*dims, batch);
  if (ws_bytes < B.total) return fail(SD_ENOSPC, "workspace %zu < %zu bytes", ws_bytes, B.total);
  for (int i = 0; i < n_layers; ++i) {
    const sd_layer& l = layers[i];
    if (!aligned(l.attn_norm) || !aligned(l.mlp_norm))
      return fail(SD_EINVAL, "layer %d: null or misaligned norm weights", i);
    if (mc) {
      if (!aligned(l.w_qkv_m) || !aligned(l.w_o_m) || !aligned(l.w_gate_m) ||
          !aligned(l.w_up_m) || !aligned(l.w_down_m))
        return fail(SD_EINVAL, "layer %d: SD_MATRIX_CORES needs the five tile weights", i);
    } else if (!aligned(l.w_qkv) || !aligned(l.w_o) || !aligned(l.w_gate) || !aligned(l.w_up) ||
               !aligned(l.w_down_t)) {
      return fail(SD_EINVAL, "layer %d: null or misaligned weight", i);
    }
    if (std::isnan(l.cats_threshold)) return fail(SD_EINVAL, "layer %d: threshold is NaN", i);
    if (l.mask_out && !aligned(l.mask_out))
      return fail(SD_EINVAL, "layer %d: misaligned mask_out", i);
    for (int b = 0; b < batch; ++b) {
      const sd_seq_kv& c = kv[(size_t)b * n_layers + i];
      if (!aligned(c.k_full) || !aligned(c.v_full))
        return fail(SD_EINVAL, "sequence %d layer %d: null or misaligned cache", b, i);
      if (c.n_full < 0 || c.n_full >= c.cap_full)
        return fail(SD_ENOSPC, "sequence %d layer %d: full cache has no free row", b, i);
      if (c.k_sel || c.v_sel) {
        if (!aligned(c.k_sel) || !aligned(c.v_sel))
          return fail(SD_EINVAL, "sequence %d layer %d: misaligned gathered buffer", b, i);
        if (c.n_sel < 0 || c.n_sel >= c.cap_sel)
          return fail(SD_ENOSPC, "sequence %d layer %d: gathered buffer has no free row", b, i);
      } else if (kv_sparse) {
        return fail(SD_EINVAL, "sequence %d layer %d: KV-sparse mode needs a gathered buffer",
                    b, i);
      }
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* wsb = static_cast<char*>(ws);
  const int d = dims->d_model, hq = dims->n_q_heads, dh = dims->head_dim, hkv = dims->n_kv_heads;
  const int ff = dims->d_ff, qkv_out = (hq + 2 * hkv) * dh;
  const float scale = 1.0f / std::sqrt((float)dh);
  float* qkv = reinterpret_cast<float*>(wsb + B.qkv);
  float* q = reinterpret_cast<float*>(wsb + B.q);
  float* attn = reinterpret_cast<float*>(wsb + B.attn);
  unsigned* mm_tickets = reinterpret_cast<unsigned*>(wsb + B.mm_tickets);
  // one matrix-core projection of the batch (tile weights w0, and w1 for up)
  auto mm = [&](int kind, const float* x, int d_in, const float* norm, const void* w0,
                const void* w1, int rows, int epi, float* out) {
    sd::BmmaArgs m{};
    m.kind = kind;
    m.x = x;
    m.nb = batch;
    m.d_in = d_in;
    m.norm = norm;
    m.eps = dims->rms_eps;
    m.w0 = w0;
    m.w1 = w1;
    m.rows = rows;
    m.epi = epi;
    m.out = out;
    m.part = reinterpret_cast<float*>(wsb + B.mm_part);
    m.ssq = reinterpret_cast<float*>(wsb + B.mm_ssq);
    m.tickets = mm_tickets;
    return m;
  };
  if (mc) sd::launch_teal_zero(mm_tickets, B.mm_groups, s);  // every launch leaves them zero
  // 128-dim heads make each 128-row group of W_qkv one head, so the matrix-core
  // QKV applies RoPE and appends to bf16 caches itself
  const bool fused_rope = mc && dh == 128 && dims->kv_dtype == SD_BF16;
  const bool fused_merge = mc && dh == 128;  // O merges the attention's split partials
  float2* rope_cs = reinterpret_cast<float2*>(wsb + B.rope);
  if (fused_rope && dims->rope_theta > 0.f) {  // the positions are the same in every layer
    sd::BatchKv at{};
    for (int b = 0; b < batch; ++b) at.pos[b] = pos[b];
    sd::launch_brope_table(at, batch, dh, dims->rope_theta, rope_cs, s);
  }
  for (int i = 0; i < n_layers; ++i) {
    const sd_layer& l = layers[i];
    // QKV for every sequence from one read of W_qkv, then RoPE and the appends
    sd::BatchKv kvs{};
    for (int b = 0; b < batch; ++b) {
      const sd_seq_kv& c = kv[(size_t)b * n_layers + i];
      kvs.pos[b] = pos[b];
      kvs.k_full[b] = c.k_full;
      kvs.v_full[b] = c.v_full;
      kvs.k_sel[b] = c.k_sel;
      kvs.v_sel[b] = c.k_sel ? c.v_sel : nullptr;
      kvs.cap_full[b] = c.cap_full;
      kvs.row_full[b] = c.n_full;
      kvs.cap_sel[b] = c.cap_sel;
      kvs.row_sel[b] = c.n_sel;
    }
    sd::BgemvArgs g{};
    if (mc && fused_rope) {  // RoPE and the appends in the last slice's epilogue
      sd::BmmaArgs m = mm(sd::K_BATCH_QKV, hidden, d, l.attn_norm, l.w_qkv_m, nullptr, qkv_out,
                          sd::MM_QKV, qkv);
      m.kvs = kvs;
      m.rope_cs = rope_cs;
      m.q_out = q;
      m.h_q = hq;
      m.h_kv = hkv;
      m.theta = dims->rope_theta;
      sd::launch_bmma(m, s);
    } else {
      if (mc) {
        sd::launch_bmma(mm(sd::K_BATCH_QKV, hidden, d, l.attn_norm, l.w_qkv_m, nullptr, qkv_out,
                           sd::MM_STORE, qkv),
                        s);
      } else {
        g.kind = sd::K_BATCH_QKV;
        g.x = hidden;
        g.nb = batch;
        g.d_in = d;
        g.norm = l.attn_norm;
        g.eps = dims->rms_eps;
        g.w = l.w_qkv;
        g.rows = qkv_out;
        g.mode = 0;
        g.out = qkv;
        sd::launch_bgemv(g, dims->w_dtype, s);
      }
      sd::launch_brope_append(qkv, batch, qkv_out, hq, hkv, dh, dims->rope_theta, kvs, q,
                              dims->kv_dtype, s);
    }
    // attention: one launch over every sequence's own cache (full or
    // gathered), chunks planned over all sequences' rows, then one merge (on
    // the matrix-core path with 128-dim heads the O projection merges the
    // split partials itself)
    int m_stride = 0, m_splits[sd::kMaxBatch] = {};
    {
      sd::AttnArgs a{};
      a.q = q;
      a.h_q = hq;
      a.h_kv = hkv;
      a.dh = dh;
      a.scale = scale;
      a.out = attn;
      a.pm = reinterpret_cast<float*>(wsb + B.pm);
      a.pl = reinterpret_cast<float*>(wsb + B.pl);
      a.pacc = reinterpret_cast<float*>(wsb + B.pacc);
      a.batched = batch;
      long long total = 0;
      int rows[sd::kMaxBatch];
      for (int b = 0; b < batch; ++b) {
        const sd_seq_kv& c = kv[(size_t)b * n_layers + i];
        a.bt.k[b] = kv_sparse ? c.k_sel : c.k_full;
        a.bt.v[b] = kv_sparse ? c.v_sel : c.v_full;
        a.bt.cap[b] = kv_sparse ? c.cap_sel : c.cap_full;
        rows[b] = (kv_sparse ? c.n_sel : c.n_full) + 1;
        a.bt.rows[b] = rows[b];
        total += (long long)hkv * rows[b];
      }
      plan_batch_splits(rows, batch, hkv, total, a.bt);
      a.n_splits = 0;
      for (int b = 0; b < batch; ++b) a.n_splits = std::max(a.n_splits, a.bt.splits[b]);
      a.n_ctx = rows[0];
      a.chunk = a.bt.chunk[0];
      a.cap = a.bt.cap[0];
      a.k = a.bt.k[0];
      a.v = a.bt.v[0];
      a.sink = a.n_ctx;
      a.no_merge = fused_merge;
      sd::launch_attn(a, dims->kv_dtype, s);
      m_stride = a.n_splits;
      for (int b = 0; b < batch; ++b) m_splits[b] = a.bt.splits[b];
    }
    uint8_t* uni = l.mask_out ? l.mask_out : reinterpret_cast<uint8_t*>(wsb + B.uni);
    float* hmid = reinterpret_cast<float*>(wsb + B.hmid);
    if (mc) {
      // O with the residual; gate and up with the CATS gate, the union and
      // hmid; down with the residual (hmid is zero where a sequence dropped
      // the channel)
      if (fused_merge) {
        sd::BmmaArgs m = mm(sd::K_BATCH_O, attn, hq * dh, nullptr, l.w_o_m, nullptr, d,
                            sd::MM_OMERGE, hidden);
        m.h_q = hq;
        m.pm = reinterpret_cast<float*>(wsb + B.pm);
        m.pl = reinterpret_cast<float*>(wsb + B.pl);
        m.pacc = reinterpret_cast<float*>(wsb + B.pacc);
        m.m_stride = m_stride;
        for (int b = 0; b < batch; ++b) m.m_splits[b] = m_splits[b];
        sd::launch_bmma(m, s);
      } else {
        sd::launch_bmma(mm(sd::K_BATCH_O, attn, hq * dh, nullptr, l.w_o_m, nullptr, d,
                           sd::MM_RESID, hidden),
                        s);
      }
      sd::BmmaArgs m = mm(sd::K_BATCH_GATE_UP, hidden, d, l.mlp_norm, l.w_gate_m, l.w_up_m, ff,
                          sd::MM_SWIGLU, nullptr);
      m.t = mlp_sparse ? l.cats_threshold : -1.0f;
      m.act = reinterpret_cast<float*>(wsb + B.act);
      m.keep = reinterpret_cast<uint8_t*>(wsb + B.keep);
      m.hmid = hmid;
      m.uni = uni;
      sd::launch_bmma(m, s);
      sd::launch_bmma(mm(sd::K_BATCH_DOWN, hmid, ff, nullptr, l.w_down_m, nullptr, d,
                         sd::MM_RESID, hidden),
                      s);
      continue;
    }
    // O with the residual, for every sequence from one read of W_o
    g = sd::BgemvArgs{};
    g.kind = sd::K_BATCH_O;
    g.x = attn;
    g.nb = batch;
    g.d_in = hq * dh;
    g.w = l.w_o;
    g.rows = d;
    g.mode = 1;
    g.out = hidden;
    sd::launch_bgemv(g, dims->w_dtype, s);
    // CATS gate per sequence, the union, the union's up rows
    g = sd::BgemvArgs{};
    g.kind = sd::K_BATCH_GATE_UP;
    g.x = hidden;
    g.nb = batch;
    g.d_in = d;
    g.norm = l.mlp_norm;
    g.eps = dims->rms_eps;
    g.w = l.w_gate;
    g.rows = ff;
    g.mode = 2;
    g.w_up = l.w_up;
    g.t = mlp_sparse ? l.cats_threshold : -1.0f;
    g.act = reinterpret_cast<float*>(wsb + B.act);
    g.keep = reinterpret_cast<uint8_t*>(wsb + B.keep);
    g.uni = uni;
    g.hmid = hmid;
    sd::launch_bgemv(g, dims->w_dtype, s);
    // down over the union for every sequence, then h_b += y_b
    sd::DownArgs da{};
    da.w_down_t = l.w_down_t;
    da.d = d;
    da.dff = ff;
    da.keep = uni;
    da.hmid = hmid;
    da.partials = reinterpret_cast<float*>(wsb + B.part);
    da.y = hidden;
    da.accumulate = 1;
    da.nb = batch;
    sd::launch_down(da, dims->w_dtype, s);
  }
  st = check_launch("sd_decode_step_batch");
  if (st) return st;
  for (int b = 0; b < batch; ++b)
    for (int i = 0; i < n_layers; ++i) {
      sd_seq_kv& c = kv[(size_t)b * n_layers + i];
      c.n_full += 1;
      if (c.k_sel) c.n_sel += 1;
    }
  return SD_OK;
}

size_t sd_calibrate_workspace_bytes(const sd_dims* dims, int32_t n_states) {
  if (check_dims(dims) != SD_OK || n_states < 1) return 0;
  const Layout L = make_layout(*dims, 0, 0);
  return L.total + (((size_t)n_states * dims->d_ff * 4 + 255) & ~size_t(255));
}

sd_status sd_cats_calibrate(const sd_dims* dims, const float* states, int32_t n_states,
                            const float* norm_w, const void* w_gate, float sparsity,
                            float* threshold, void* ws, size_t ws_bytes, void* stream) {
  sd_status st = check_dims(dims);
  if (st) return st;
  if (!aligned(states) || !aligned(w_gate) || !threshold || !aligned(ws) ||
      (norm_w && !aligned(norm_w)))
    return fail(SD_EINVAL, "null or misaligned pointer");
  if (n_states < 1) return fail(SD_EINVAL, "n_states must be >= 1");
  if (!(sparsity >= 0.f && sparsity <= 1.f)) return fail(SD_EINVAL, "sparsity outside [0, 1]");
  const size_t need = sd_calibrate_workspace_bytes(dims, n_states);
  if (ws_bytes < need) return fail(SD_ENOSPC, "workspace %zu < %zu bytes", ws_bytes, need);
  const Layout L = make_layout(*dims, 0, 0);
  char* wsb = static_cast<char*>(ws);
  float* vals = reinterpret_cast<float*>(wsb + L.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  sd::GateArgs g{};
  g.x = states;
  g.norm = norm_w;
  g.eps = dims->rms_eps;
  g.w_gate = w_gate;
  g.calib = 1;
  g.d = dims->d_model;
  g.dff = dims->d_ff;
  g.t = -1.f;
  g.store_abs = 1;
  g.act = vals;
  g.n_states = n_states;
  sd::launch_gate(g, dims->w_dtype, s);
  const size_t N = (size_t)n_states * dims->d_ff;
  const size_t k = (size_t)std::floor((double)sparsity * (double)N + 0.5);
  sd::launch_kth_smallest(vals, N, k, reinterpret_cast<unsigned*>(wsb + L.kth_hist),
                          reinterpret_cast<unsigned*>(wsb + L.kth_state), threshold, s);
  return check_launch("sd_cats_calibrate");
}

}  // extern "C"
