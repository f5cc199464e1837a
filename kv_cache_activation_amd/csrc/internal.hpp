// Host-side launchers shared between the kernels and the C ABI layer.
// All launchers enqueue on `s` and return without synchronizing; the caller
// checks hipGetLastError() afterwards.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sd.h"

namespace sd {

// Kernel kinds for the opt-in profiler (order = names in profile.cpp).
enum KernelKind {
  K_QKV, K_ATTN_PARTIAL, K_ATTN_COMBINE, K_O, K_GATE_UP, K_DOWN, K_MLP_REDUCE, K_SEL_LSE,
  K_SEL_LSE_FINAL, K_SEL_SCORE, K_SEL_TOPK, K_SEL_GATHER, K_KTH, K_MASKED_SCORES,
  K_MASKED_SOFTMAX, K_MASKED_PV, K_TEAL_QKV, K_TEAL_ZERO, K_TEAL_O, K_TEAL_GATE_UP,
  K_TEAL_DOWN, K_BATCH_QKV, K_BATCH_ROPE, K_BATCH_O, K_BATCH_GATE_UP, K_BATCH_DOWN,
  K_PACK_TILES, K_COUNT
};

// Start/stop events of one launch of kind `kind` while profiling is on (both
// null otherwise, or for kind < 0).  The events are attached to the dispatch
// itself, so they time the kernel's execution, not the queue around it.
struct ProfEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
ProfEvents prof_events(int kind);

// Every kernel of the library is launched through here.
template <typename F, typename... Args>
inline void launch_kernel(int kind, F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s,
                          Args... args) {
  const ProfEvents e = prof_events(kind);
  hipExtLaunchKernelGGL(kernel, grid, block, lds, s, e.start, e.stop, 0u, args...);
}

// One int per KV head (ragged per-head budgets), passed by value.
constexpr int kMaxKvHeads = 32;
struct HeadInts {
  int v[kMaxKvHeads];
};

// cos and sin of the rotation angle of each RoPE pair index (d_h / 2 <= 64)
struct RopeTable {
  float c[64];
  float s[64];
};

struct QkvArgs {
  const float* h;
  const float* norm;
  float eps;
  const void* w;
  int d, h_q, h_kv, dh;
  RopeTable rope;
  float* q_out;
  void* k_full;
  void* v_full;
  int cap_full, row_full;
  void* k_sel;
  void* v_sel;
  int cap_sel, row_sel;
  int ragged;          // the gathered buffer's row per KV head is sel_rows.v[kv]
  HeadInts sel_rows;
};

struct GateArgs {
  const float* x;
  const float* norm;  // nullptr: x is used as is
  float eps;
  const void* w_gate;
  const void* w_up;   // nullptr: no up projection
  int d, dff;
  float t;
  int gate_in, store_abs, calib;
  float* act;
  uint8_t* keep;      // nullptr: activations only (calibration)
  float* hmid;        // a_i (W_up[i] . x) for kept channels
  int n_states;       // batched gate for calibration; 1 otherwise
};

// Down projection over the kept channels: the kept list is split into P
// equal slices (P = down_parts(d_ff) workgroups, each at most kDownList
// channels).
constexpr int kDownList = 64;
constexpr int kDownMinParts = 256;
constexpr int kDownMaxParts = 512;  // d_ff <= kDownList * kDownMaxParts
int down_parts(int dff);

struct DownArgs {
  const void* w_down_t;
  int d, dff;
  const uint8_t* keep;
  const float* hmid;
  float* partials;     // [down_parts(dff), d]
  float* y;
  int accumulate;      // y += result instead of y = result
  int32_t* idx_out;    // optional ascending kept list
  int32_t* n_kept_out; // optional
  int nb;              // sequences sharing the rows (0 or 1: one); hmid [nb, dff], y [nb, d]
};

// TEAL projection over column blocks: y = sum over kept inputs j (|x_j| > t,
// after the optional RMSNorm) of x_j w[j, :], the weight stored in blocks of
// kTealBlock output columns, w_blk [nblk][d_in][kTealBlock] (nblk =
// ceil(d_out / kTealBlock), padding columns past d_out never written out).
// Grid (slices, blocks): slice s takes the input channels [s R, (s + 1) R)
// of the input, block b the columns [b kTealBlock, (b + 1) kTealBlock); the
// last slice of a block to finish adds the slices' partial sums and applies
// the epilogue.
constexpr int kTealBlock = 128;
constexpr int kTealMaxRange = 2048;  // input channels per slice, at most
constexpr int kTealMaxSlices = 32;
constexpr int kTealMaxBlocks = 1024; // blocks' tickets in the workspace
// TEAL_DOWN and TEAL_CATS_DOWN are TEAL_ACC under kernel names of their own:
// the down projection after TEAL's gate and up, and after the CATS gate (or a
// dense one), so that traces and counters tell them from the O projection.
enum TealEpi {
  TEAL_STORE = 0,
  TEAL_ACC = 1,
  TEAL_SWIGLU = 2,
  TEAL_QKV = 3,
  TEAL_DOWN = 4,
  TEAL_CATS_DOWN = 5
};
int teal_slices(int d_in, int d_out);

struct TealArgs {
  int kind;            // profiler kind of this projection
  const float* x;
  int d_in;
  const float* norm;   // nullptr: no RMSNorm
  float eps, t;        // t < 0: keep every channel
  const void* w0;      // column blocks [nblk][d_in][kTealBlock]
  const void* w1;      // optional second matrix with the same input (gate and up)
  int d_out;
  float* part;         // [slices, nblk kTealBlock] per matrix (w1's after w0's)
  unsigned* tickets;   // [nblk]: zero before the launch, zero again after it
  int epi;             // TealEpi
  float* y;            // STORE / ACC: the outputs of w0; SWIGLU: SiLU(y0) * y1
  float* y2;           // STORE / ACC with w1: its outputs
  float t_next;        // SWIGLU: the next projection's threshold, for
  uint8_t* keep_next;  //   keep_next[c] = |SiLU(y0) y1| > t_next (t_next < 0: all)
  QkvArgs qkv;         // QKV: RoPE table, q out, cache appends (qkv.h unused)
  int32_t* idx_out;    // optional ascending kept list
  int32_t* n_kept_out; // optional
  uint8_t* keep_out;   // optional keep bytes [d_in]
};

// Batched attention: sequence s has its own cache (k[s], v[s], cap[s]) of
// rows[s] valid rows per KV head, split into splits[s] chunks of chunk[s]
// rows; a flat grid where sequence s owns blocks [starts[s], starts[s+1])
// (entries past the last sequence hold INT_MAX).
struct AttnBatch {
  const void* k[8];
  const void* v[8];
  int cap[8], rows[8], chunk[8], splits[8], starts[8];
};

struct AttnArgs {
  const float* q;
  const void* k;
  const void* v;
  int cap, n_ctx, h_q, h_kv, dh;
  int sink, shift;      // logical row j reads physical row j + (j >= sink ? shift : 0)
  int per_query_head;   // one workgroup per query head (no K/V sharing across a group)
  int ragged;           // KV head kv has lens.v[kv] rows (n_ctx is their maximum)
  HeadInts lens;
  int batched;          // > 0: that many sequences, described by bt (q, out: [nb, h_q, d_h])
  AttnBatch bt;
  float scale;
  int n_splits, chunk;
  float* pm;
  float* pl;
  float* pacc;
  float* out;
  float* lse;
  int no_merge;         // leave the split partials for the consumer (no merge launch)
};

struct SelectArgs {
  const void* k;
  const void* v;
  int cap_full, n;
  const float* q_win;
  int w, n_sink, k_keep, h_q, h_kv, dh;
  float* scores;
  int32_t* idx;
  void* k_sel;
  void* v_sel;
  int cap_sel;
  int chunk, n_chunks;
  float* lse_part;   // [h_kv, n_chunks, G*w, 2]
  float* lse;        // [h_q, w] (log2 domain)
  int skip_scoring;
  int ragged;        // per-head budgets k_heads (k_keep unused), idx rows of idx_stride
  HeadInts k_heads;
  int idx_stride;
  unsigned* topk_ws; // chunked top-k: topk_ws_words(h_kv) words, or null for one workgroup per head
};

// Chunked top-k over long contexts: at most kTopkMaxChunks chunks per KV head.
constexpr int kTopkMaxChunks = 64;
inline size_t topk_ws_words(int h_kv) { return (size_t)h_kv * (kTopkMaxChunks * (256 + 2) + 2); }

// Batched decode (nb sequences sharing the weight reads): the sequences'
// positions and caches, passed by value.
constexpr int kMaxBatch = 8;
struct BatchKv {
  int pos[kMaxBatch];
  void* k_full[kMaxBatch];
  void* v_full[kMaxBatch];
  void* k_sel[kMaxBatch];   // nullptr: no gathered buffer
  void* v_sel[kMaxBatch];
  int cap_full[kMaxBatch], row_full[kMaxBatch], cap_sel[kMaxBatch], row_sel[kMaxBatch];
};

// Batched GEMV y[b] = W x_b, W [rows, d_in] row-major, x [nb, d_in]
// (d_in <= 4096, a multiple of 8); mode 0 store out [nb, rows], 1 out +=,
// 2 the CATS gate with the up rows of the union (act, keep, hmid [nb, rows],
// uni [rows]).
struct BgemvArgs {
  int kind;
  const float* x;
  int nb, d_in;
  const float* norm;  // nullptr: x as is
  float eps;
  const void* w;
  int rows, mode;
  float* out;
  const void* w_up;
  float t;
  float* act;
  uint8_t* keep;
  uint8_t* uni;
  float* hmid;
};
void launch_bgemv(const BgemvArgs& a, int w_dtype, hipStream_t s);
// cs[b][i] = (cos, sin) of rotation pair i at sequence b's position (the
// rotation of launch_brope_append), for b < nb and i < dh / 2.
void launch_brope_table(const BatchKv& kvs, int nb, int dh, float theta, float2* cs,
                        hipStream_t s);
void launch_brope_append(const float* qkv, int nb, int qkv_out, int h_q, int h_kv, int dh,
                         float theta, const BatchKv& kvs, float* q, int kv_dtype, hipStream_t s);
int cu_count_dev();

// Batched projections on the matrix cores, weights in 16-row x 32-channel
// tiles (A-operand order of v_mfma_f32_16x16x32_bf16, bf16 only).  Grid
// (input slices, bmma_groups row groups of 128 rows); the last
// slice of a row group to finish sums the slices' partials and applies the
// epilogue.
enum { MM_STORE = 0, MM_RESID = 1, MM_SWIGLU = 2, MM_QKV = 3, MM_OMERGE = 4 };
struct BmmaArgs {
  int kind;
  const float* x;      // [nb, d_in] float32 (d_in % 8 == 0)
  int nb, d_in;
  const float* norm;   // RMSNorm weights [d_in], or nullptr
  float eps;
  const void* w0;      // tiles of W [rows, d_in]
  const void* w1;      // MM_SWIGLU: tiles of W_up (same shape); nullptr otherwise
  int rows, epi;
  float* out;          // MM_STORE: out = y; MM_RESID: out += y ([nb, rows])
  float t;             // MM_SWIGLU: CATS threshold (t < 0 keeps every channel)
  float* act;          // MM_SWIGLU outputs [nb, rows]: SiLU(gate), keep bytes, hmid,
  uint8_t* keep;       //   and the union uni [rows]
  float* hmid;
  uint8_t* uni;
  float* part;         // bmma_part_floats(rows, d_in, w1 != nullptr)
  float* ssq;          // bmma_ssq_floats(...) (with a norm)
  unsigned* tickets;   // [bmma_groups(rows)]: zero before the launch, zero after it
  // MM_QKV (head_dim 128, bf16 caches: row group g is head g): RoPE at each
  // sequence's position on q and k (rope_cs from launch_brope_table; theta
  // <= 0: none), q written to q_out [nb, h_q, 128], k and v appended to each
  // sequence's caches (as launch_brope_append)
  BatchKv kvs;
  const float2* rope_cs;
  float* q_out;
  int h_q, h_kv;
  float theta;
  // MM_OMERGE (O with the residual, head_dim 128): x is not read; sequence b's
  // input is merged from the batched attention's split partials of its h_q
  // heads (pm, pl, pacc with stride m_stride splits, m_splits[b] of them)
  const float* pm;
  const float* pl;
  const float* pacc;
  int m_stride;
  int m_splits[kMaxBatch];
};
int bmma_groups(int rows);
size_t bmma_part_floats(int rows, int d_in, bool dual);
size_t bmma_ssq_floats(int rows, int d_in, bool dual);
void launch_bmma(const BmmaArgs& a, hipStream_t s);
// W [rows, d_in] bf16 row-major (d_in % 8 == 0) -> the tile layout
void launch_pack_tiles(const void* w, int rows, int d_in, void* out, hipStream_t s);

void launch_qkv(const QkvArgs& a, int w_dtype, int kv_dtype, hipStream_t s);
void launch_o(const float* attn, const void* w, int din, int dout, float* h, int w_dtype,
              hipStream_t s);
void launch_gate(const GateArgs& a, int w_dtype, hipStream_t s);
void launch_down(const DownArgs& a, int w_dtype, hipStream_t s);
void launch_teal(const TealArgs& a, int w_dtype, int kv_dtype, hipStream_t s);
// zero n ticket words (before the first TEAL projection of a call)
void launch_teal_zero(unsigned* tickets, int n, hipStream_t s);
void launch_attn(const AttnArgs& a, int kv_dtype, hipStream_t s);
// Masked dense attention over every allocated row (rows >= n_ctx masked): scores
// of each query head into `scores` [h_q, cap], a row softmax, then P.V in
// n_splits chunks summed in order.  A deliberately plain comparison path.
void launch_attn_masked(const AttnArgs& a, float* scores, int kv_dtype, hipStream_t s);
void launch_select(const SelectArgs& a, int kv_dtype, hipStream_t s);
// k-th smallest (1-based k) of n non-negative float32 values; writes the value
// to *out (or -1 when k == 0).  hist: 256 uint32 scratch words; state: 4 words.
void launch_kth_smallest(const float* vals, size_t n, size_t k, unsigned* hist, unsigned* state,
                         float* out, hipStream_t s);

// One read of bytes (a multiple of 8192) of buf; out[SD_STREAM_BLOCKS] XOR checksums.
void launch_stream_read(const void* buf, size_t bytes, unsigned* out, hipStream_t s);

// Records a message for sd_last_error() on the calling thread; returns st.
sd_status set_error(sd_status st, const char* msg);

}  // namespace sd
