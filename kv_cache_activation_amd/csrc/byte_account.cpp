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
                                     double fixed_bytes, const sd_latency_model* lat,
                                     sd_byte_record* out) {
  if (!dims || !out || n_layers < 1 || !(n >= 0) || !(r_p >= 0 && r_p <= 1) ||
      !(r_kv >= 0 && r_kv <= 1) || !(s_w > 0) || !(s_kv > 0) || !(fixed_bytes >= 0))
    return SD_EINVAL;
  if (dims->d_model < 1 || dims->n_q_heads < 1 || dims->n_kv_heads < 1 || dims->head_dim < 1 ||
      dims->d_ff < 1)
    return SD_EINVAL;
  if (lat && !(lat->bw_eff > 0 && std::isfinite(lat->bw_eff) && std::isfinite(lat->c_p) &&
               std::isfinite(lat->c_kv)))
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
  const double inf = std::numeric_limits<double>::infinity();
  const double nan = std::numeric_limits<double>::quiet_NaN();
  // the projection branch's saving per layer, in cache tokens
  const double p_tokens = sparse_params * s_w * (1.0 - r_p) / per_token_kv;
  out->b_attn = attn_params * s_w;
  out->b_mlp = mlp_params * s_w;
  out->b_kv = per_token_kv * n;
  out->b_total = n_layers * (out->b_attn + out->b_mlp + out->b_kv) + fixed_bytes;
  out->delta_p = n_layers * sparse_params * s_w * (1.0 - r_p);
  out->delta_kv = n_layers * out->b_kv * (1.0 - r_kv);
  out->bound_p = out->b_total / (out->b_total - out->delta_p);
  out->bound_kv = out->b_total / (out->b_total - out->delta_kv);
  out->bound_both = out->b_total / (out->b_total - out->delta_p - out->delta_kv);
  out->n_star = r_kv < 1.0 ? p_tokens / (1.0 - r_kv) : inf;
  // a KV method with a fixed budget b skips (n - b) tokens: it matches the
  // projection branch at n = b + p_tokens (§3.3, r_kv = b / n substituted)
  out->n_star_budget = r_kv * n + p_tokens;
  if (lat) {
    // §4.3: s is the byte time of the cache rows the KV branch skips per 1K
    // tokens; a kernel-cost difference c_p - c_kv moves the crossing by
    // (c_p - c_kv) / s thousand tokens
    out->gap_per_k = n_layers * per_token_kv * 1024.0 * (1.0 - r_kv) / lat->bw_eff;
    out->n_lat = r_kv < 1.0 ? out->n_star - (lat->c_p - lat->c_kv) / out->gap_per_k * 1024.0
                            : inf;
  } else {
    out->gap_per_k = nan;
    out->n_lat = nan;
  }
  return SD_OK;
}

// The latency model of a measured sweep (§4.3): time = bytes / bw_eff + c.
// bw_eff comes from the dense step alone (the mode whose time grows fastest
// with context); each branch's cost is its mean excess over byte time.
extern "C" sd_status sd_latency_fit(int32_t n_points, const double* bytes_dense,
                                    const double* t_dense, int32_t n_modes,
                                    const double* bytes_modes, const double* t_modes,
                                    double* bw_eff, double* c_modes) {
  if (n_points < 2 || !bytes_dense || !t_dense || !bw_eff || n_modes < 0 ||
      (n_modes > 0 && (!bytes_modes || !t_modes || !c_modes)))
    return SD_EINVAL;
  double bm = 0, tm = 0;
  for (int32_t i = 0; i < n_points; ++i) {
    if (!std::isfinite(bytes_dense[i]) || !std::isfinite(t_dense[i])) return SD_EINVAL;
    bm += bytes_dense[i];
    tm += t_dense[i];
  }
  bm /= n_points;
  tm /= n_points;
  double sbb = 0, sbt = 0;
  for (int32_t i = 0; i < n_points; ++i) {
    const double db = bytes_dense[i] - bm;
    sbb += db * db;
    sbt += db * (t_dense[i] - tm);
  }
  if (!(sbb > 0) || !(sbt > 0)) return SD_EINVAL;
  const double bw = sbb / sbt;  // bytes per second
  for (int32_t m = 0; m < n_modes; ++m) {
    double c = 0;
    for (int32_t i = 0; i < n_points; ++i) {
      const double b = bytes_modes[(size_t)m * n_points + i], t = t_modes[(size_t)m * n_points + i];
      if (!std::isfinite(b) || !std::isfinite(t)) return SD_EINVAL;
      c += t - b / bw;
    }
    c_modes[m] = c / n_points;
  }
  *bw_eff = bw;
  return SD_OK;
}

extern "C" sd_status sd_latency_crossing(int32_t n_points, const double* ctx, const double* t_a,
                                         const double* t_b, double* n_cross) {
  if (n_points < 1 || !ctx || !t_a || !t_b || !n_cross) return SD_EINVAL;
  for (int32_t i = 0; i < n_points; ++i) {
    if (!std::isfinite(ctx[i]) || !std::isfinite(t_a[i]) || !std::isfinite(t_b[i]))
      return SD_EINVAL;
    if (i > 0 && !(ctx[i] > ctx[i - 1])) return SD_EINVAL;
  }
  for (int32_t i = 0; i < n_points; ++i) {
    const double di = t_a[i] - t_b[i];
    if (di == 0.0) {
      *n_cross = ctx[i];
      return SD_OK;
    }
    if (i + 1 < n_points) {
      const double dn = t_a[i + 1] - t_b[i + 1];
      if (dn != 0.0 && ((di < 0.0) != (dn < 0.0))) {
        // the zero of the straight line through (ctx[i], di) and (ctx[i+1], dn)
        *n_cross = ctx[i] + (ctx[i + 1] - ctx[i]) * di / (di - dn);
        return SD_OK;
      }
    }
  }
  *n_cross = std::numeric_limits<double>::quiet_NaN();
  return SD_OK;
}

extern "C" sd_status sd_latency_gate(int32_t n_configs, const double* t_step,
                                     const double* t_once, const uint8_t* admissible,
                                     double horizon, int32_t* best) {
  if (n_configs < 1 || !t_step || !t_once || !best || !(horizon >= 0) || !std::isfinite(horizon))
    return SD_EINVAL;
  for (int32_t i = 0; i < n_configs; ++i)
    if (!(t_step[i] >= 0) || !(t_once[i] >= 0) || !std::isfinite(t_step[i]) ||
        !std::isfinite(t_once[i]))
      return SD_EINVAL;
  int32_t b = -1;
  double bt = 0;
  for (int32_t i = 0; i < n_configs; ++i) {
    if (admissible && !admissible[i]) continue;
    const double tot = horizon * t_step[i] + t_once[i];
    if (b < 0 || tot < bt) {  // strict: equal totals keep the lower index
      b = i;
      bt = tot;
    }
  }
  *best = b;
  return SD_OK;
}

// Batched crossover ([Cross] §3.3, "Dispatch and batching"): B sequences share
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
  const sd_status st =
      sd_byte_account(dims, 1, 0.0, 0.0, r_kv, s_w, s_kv, proj_set, 0.0, nullptr, &rec);
  if (st != SD_OK) return st;
  const double sparse_bytes = rec.delta_p;  // P s_w
  const double per_token_kv = 2.0 * dims->n_kv_heads * dims->head_dim * s_kv;
  *n_star = r_kv < 1.0 ? sparse_bytes * (1.0 - u_b) / (batch * per_token_kv * (1.0 - r_kv))
                       : std::numeric_limits<double>::infinity();
  return SD_OK;
}
