// Byte account of one decode step ("Where Activation Sparsity and KV-Cache
// Sparsity Cross in LLM Decoding", §3).  Host only.
//
// Per layer a step reads the four attention projections (q, k, v fused; o),
// the three feed-forward projections and the keys and values of n cached
// tokens.  The projection branch keeps a fraction r_p of the channels of its
// projection set and skips the rest of those weights (constant in n); the KV
// branch reads a fraction r_kv of the cache (savings linear in n).  A purely
// bandwidth-bound step that skips dB of B bytes is at most B / (B - dB) times
// faster, and the crossover n* is the context at which both savings match.
#include <cmath>
#include <limits>

#include "../../include/sd.h"

extern "C" sd_status sd_byte_account(const sd_dims* dims, int32_t n_layers, double n, double r_p,
                                     double r_kv, double s_w, double s_kv, int32_t proj_set,
                                     double fixed_bytes, sd_byte_record* out) {
  if (!dims || !out || n_layers < 1 || !(n >= 0) || !(r_p >= 0 && r_p <= 1) ||
      !(r_kv >= 0 && r_kv <= 1) || !(s_w > 0) || !(s_kv > 0) || !(fixed_bytes >= 0))
    return SD_EINVAL;
  if (dims->d_model < 1 || dims->n_q_heads < 1 || dims->n_kv_heads < 1 || dims->head_dim < 1 ||
      dims->d_ff < 1)
    return SD_EINVAL;
  const double d = dims->d_model, hq = dims->n_q_heads, hkv = dims->n_kv_heads,
               dh = dims->head_dim, ff = dims->d_ff;
  const double attn_params = d * (hq * dh + 2.0 * hkv * dh) + hq * dh * d;
  const double mlp_params = 3.0 * d * ff;
  double sparse_params;
  switch (proj_set) {
    case SD_PROJ_ALL7: sparse_params = attn_params + mlp_params; break;
    case SD_PROJ_FFN: sparse_params = mlp_params; break;
    case SD_PROJ_CATS: sparse_params = 2.0 * d * ff; break;  // CATS reads the gate densely
    default: return SD_EINVAL;
  }
  const double per_token_kv = 2.0 * hkv * dh * s_kv;  // one key and one value row
  out->b_attn = attn_params * s_w;
  out->b_mlp = mlp_params * s_w;
  out->b_kv = per_token_kv * n;
  out->b_total = n_layers * (out->b_attn + out->b_mlp + out->b_kv) + fixed_bytes;
  out->delta_p = n_layers * sparse_params * s_w * (1.0 - r_p);
  out->delta_kv = n_layers * out->b_kv * (1.0 - r_kv);
  out->bound_p = out->b_total / (out->b_total - out->delta_p);
  out->bound_kv = out->b_total / (out->b_total - out->delta_kv);
  out->bound_both = out->b_total / (out->b_total - out->delta_p - out->delta_kv);
  out->n_star = r_kv < 1.0 ? sparse_params * s_w * (1.0 - r_p) / (per_token_kv * (1.0 - r_kv))
                           : std::numeric_limits<double>::infinity();
  return SD_OK;
}

// Batched crossover ([Cross] §3.2, "Dispatch and batching"): B sequences share
// each weight read, so the projection branch skips only the channels no
// sequence keeps, a fraction 1 - u_b of its projection set, once per step,
// while the KV branch still skips (1 - r_kv) of every sequence's cache.  Per
// sequence the savings meet at n_B* = P s_w (1 - u_b) / (B 2 h_kv d_h s_kv (1 - r_kv)).
extern "C" sd_status sd_byte_crossover_batch(const sd_dims* dims, int32_t batch, double u_b,
                                             double r_kv, double s_w, double s_kv,
                                             int32_t proj_set, double* n_star) {
  if (!dims || !n_star || batch < 1 || !(u_b >= 0 && u_b <= 1) || !(r_kv >= 0 && r_kv <= 1) ||
      !(s_w > 0) || !(s_kv > 0))
    return SD_EINVAL;
  sd_byte_record rec;
  // the projection set's parameter count: the one-sequence skipped bytes at r_p = 0
  const sd_status st = sd_byte_account(dims, 1, 0.0, 0.0, r_kv, s_w, s_kv, proj_set, 0.0, &rec);
  if (st != SD_OK) return st;
  const double sparse_bytes = rec.delta_p;  // P s_w
  const double per_token_kv = 2.0 * dims->n_kv_heads * dims->head_dim * s_kv;
  *n_star = r_kv < 1.0 ? sparse_bytes * (1.0 - u_b) / (batch * per_token_kv * (1.0 - r_kv))
                       : std::numeric_limits<double>::infinity();
  return SD_OK;
}
