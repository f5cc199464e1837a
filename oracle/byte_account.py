"""Oracle: byte account of one decode step (test infrastructure only).

Follows [Cross] §3 "The Byte Crossover".  The body of §3.1 (the traffic
definitions) is missing from the extracted page; the definitions below are
the reading that the rest of §3 and the printed numbers support:

* every step reads all projection weights of every layer (§1, §3.2): the four
  attention projections W_q, W_k, W_v, W_o and the three feed-forward
  projections W_gate, W_up, W_down;
* every step reads the keys and values of all n cached tokens (§1);
* an optional fixed term (the LM head when whole-model bounds are compared
  with the page's printed bounds; zero for bare layer stacks).

Savings and bounds (§3.2, §3.3):

* projection branch keeps a fraction r_P of the channels of the projections
  in its set and saves  L * P_set * s_w * (1 - r_P)  bytes, independent of n;
* KV branch reads a fraction r_KV of the cache and saves
  L * B_KV(n) * (1 - r_KV)  bytes, linear in n;
* a purely bandwidth-bound step that removes dB of B_total bytes is at most
  B_total / (B_total - dB) times faster;
* the crossover n* equates the two savings; it scales with s_w / s_kv;
* with a fixed KV budget b (r_KV = b/n) the crossover is b + P(1-r_P)/(2 h_kv d_h)
  (bytes-per-element ratio folded in);
* a batch of B sequences that activates a union fraction u_B of the channels
  crosses at P(1-u_B)/(2 B h_kv d_h (1-r_KV));
* §4.3: with kernel costs c_P and c_KV beyond byte time, latencies cross near
  n_lat = n* - (c_P - c_KV)/s, s = time of the KV bytes the KV branch skips per
  1K tokens.

Token counts use K = 1024 tokens; bytes are plain integers (decimal MB/GB
only when printed), per §3.

Pinned by tests/test_oracle_byte_account.py against the numbers [Cross]
prints (§3.3, §4.3, §4.4, §5.2) -- see tests/golden/byte_account_pins.json.
"""

from __future__ import annotations

from dataclasses import dataclass

K_TOKENS = 1024  # [Cross] §3: "K" means 1,024 tokens.

PROJ_SETS = ("all7", "ffn", "cats")


@dataclass(frozen=True)
class Dims:
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int


def attn_proj_params(dm: Dims) -> int:
    """Parameters of W_q, W_k, W_v (fused [h_q d_h + 2 h_kv d_h, d]) and W_o."""
    qkv_out = dm.n_q_heads * dm.head_dim + 2 * dm.n_kv_heads * dm.head_dim
    return dm.d_model * qkv_out + dm.n_q_heads * dm.head_dim * dm.d_model


def mlp_params(dm: Dims) -> int:
    """Parameters of the three feed-forward projections (gate, up, down)."""
    return 3 * dm.d_model * dm.d_ff


def sparse_params(dm: Dims, proj_set: str) -> int:
    """P_set: the parameters whose reads the projection branch can skip.

    all7 -- all seven projections ([Cross] §3.2, TEAL in §4.1);
    ffn  -- the three feed-forward projections ([Cross] Table 1 caption);
    cats -- up and down only: CATS thresholds the gate output, so the gate
            itself is always read densely ([SATS], CATS runtime masking).
    """
    if proj_set == "all7":
        return attn_proj_params(dm) + mlp_params(dm)
    if proj_set == "ffn":
        return mlp_params(dm)
    if proj_set == "cats":
        return 2 * dm.d_model * dm.d_ff
    raise ValueError(f"unknown projection set {proj_set!r}")


def b_attn(dm: Dims, s_w: float) -> float:
    return attn_proj_params(dm) * s_w


def b_mlp(dm: Dims, s_w: float) -> float:
    return mlp_params(dm) * s_w


def b_kv(dm: Dims, n: float, s_kv: float) -> float:
    """Bytes of keys plus values of n cached tokens in one layer."""
    return 2.0 * n * dm.n_kv_heads * dm.head_dim * s_kv


def b_total(dm: Dims, n_layers: int, n: float, s_w: float, s_kv: float,
            fixed_bytes: float = 0.0) -> float:
    return n_layers * (b_attn(dm, s_w) + b_mlp(dm, s_w) + b_kv(dm, n, s_kv)) + fixed_bytes


def delta_p(dm: Dims, n_layers: int, r_p: float, s_w: float, proj_set: str) -> float:
    """Bytes the projection branch removes per step (constant in n)."""
    return n_layers * sparse_params(dm, proj_set) * s_w * (1.0 - r_p)


def delta_kv(dm: Dims, n_layers: int, n: float, r_kv: float, s_kv: float) -> float:
    """Bytes the KV branch removes per step (linear in n)."""
    return n_layers * b_kv(dm, n, s_kv) * (1.0 - r_kv)


def speedup_bound(total: float, removed: float) -> float:
    """Ideal speedup of a bandwidth-bound step that skips `removed` bytes
    (unbounded when nothing is left to read)."""
    left = total - removed
    return total / left if left > 0 else float("inf")


def crossover(dm: Dims, r_p: float, r_kv: float, s_w: float, s_kv: float,
              proj_set: str = "all7") -> float:
    """n*: context length (tokens) at which both savings are equal."""
    num = sparse_params(dm, proj_set) * s_w * (1.0 - r_p)
    den = 2.0 * dm.n_kv_heads * dm.head_dim * s_kv * (1.0 - r_kv)
    return num / den


def crossover_fixed_budget(dm: Dims, budget: float, r_p: float, s_w: float,
                           s_kv: float, proj_set: str = "all7") -> float:
    """n* for a KV method that keeps a fixed number `budget` of tokens."""
    per_token = 2.0 * dm.n_kv_heads * dm.head_dim * s_kv
    return budget + sparse_params(dm, proj_set) * s_w * (1.0 - r_p) / per_token


def crossover_batched(dm: Dims, batch: int, u_b: float, r_kv: float, s_w: float,
                      s_kv: float, proj_set: str = "all7") -> float:
    """n_B*: per-sequence crossover when B sequences share each weight read and
    the union of their active channels covers a fraction u_b of the weights."""
    num = sparse_params(dm, proj_set) * s_w * (1.0 - u_b)
    den = 2.0 * batch * dm.n_kv_heads * dm.head_dim * s_kv * (1.0 - r_kv)
    return num / den


def gap_growth_per_k(dm: Dims, n_layers: int, r_kv: float, s_kv: float,
                     bw_bytes_per_s: float) -> float:
    """s: seconds by which the byte-time gap grows per 1K more context tokens."""
    return n_layers * b_kv(dm, K_TOKENS, s_kv) * (1.0 - r_kv) / bw_bytes_per_s


def latency_crossing(n_star_tokens: float, c_p: float, c_kv: float,
                     s_per_k: float) -> float:
    """n_lat (tokens) = n* - (c_P - c_KV)/s with s per 1K tokens ([Cross] §4.3)."""
    return n_star_tokens - (c_p - c_kv) / s_per_k * K_TOKENS


# ------------------------------------------------- from a measured sweep (§4.3)
# The page locates its crossings from kernel costs measured on a context sweep
# (its Appendix D, which the extracted text does not hold).  The plainest
# reading: a bandwidth-bound step takes its bytes / BW_eff plus a fixed kernel
# cost, BW_eff comes from how the dense step's time grows with its bytes, and
# each branch's cost c_X is what its measured time holds beyond its byte time.

def effective_bandwidth(bytes_dense, t_dense) -> float:
    """BW_eff (bytes/s): inverse slope of the least-squares line of the dense
    step's time against its bytes over the sweep's contexts."""
    b = [float(x) for x in bytes_dense]
    t = [float(x) for x in t_dense]
    if len(b) < 2 or len(b) != len(t):
        raise ValueError("need two or more (bytes, time) points")
    bm = sum(b) / len(b)
    tm = sum(t) / len(t)
    sbb = sum((x - bm) ** 2 for x in b)
    sbt = sum((x - bm) * (y - tm) for x, y in zip(b, t))
    if sbb <= 0 or sbt <= 0:
        raise ValueError("time must grow with bytes")
    return sbb / sbt


def kernel_cost(bytes_x, t_x, bw_eff: float) -> float:
    """c_X (s): mean over the sweep of the branch's time beyond its byte time."""
    pts = list(zip(bytes_x, t_x))
    if not pts:
        raise ValueError("empty sweep")
    return sum(float(t) - float(b) / bw_eff for b, t in pts) / len(pts)


def measured_crossing(ctx, t_a, t_b) -> float:
    """Context (tokens) where the latency curves t_a and t_b cross, by linear
    interpolation of t_a - t_b between the first two neighbouring contexts
    whose differences change sign (a zero difference is itself the crossing);
    NaN when the curves do not cross inside the sweep.  `ctx` ascending."""
    n = [float(x) for x in ctx]
    dlt = [float(a) - float(b) for a, b in zip(t_a, t_b)]
    if len(n) != len(dlt) or any(x >= y for x, y in zip(n, n[1:])):
        raise ValueError("contexts must ascend, one time per context and curve")
    for i in range(len(n)):
        if dlt[i] == 0.0:
            return n[i]
        if i + 1 < len(n) and (dlt[i] < 0.0) != (dlt[i + 1] < 0.0) and dlt[i + 1] != 0.0:
            return n[i] + (n[i + 1] - n[i]) * dlt[i] / (dlt[i] - dlt[i + 1])
    return float("nan")


def latency_gate(t_step, t_once, horizon: float, admissible=None) -> int:
    """The latency gate of [Cross] §3.3 "Dispatch and batching": among the
    admissible configurations, the one with the least time for `horizon`
    decode steps, horizon * t_step plus its one-time cost (the KV selection);
    equal times go to the lower index.  -1 when none is admissible."""
    best, best_t = -1, 0.0
    for i, (ts, to) in enumerate(zip(t_step, t_once)):
        if admissible is not None and not admissible[i]:
            continue
        tot = horizon * float(ts) + float(to)
        if best < 0 or tot < best_t:
            best, best_t = i, tot
    return best


@dataclass(frozen=True)
class Record:
    """Everything the account says about one (dims, n, keep ratios) point."""
    b_attn: float
    b_mlp: float
    b_kv: float
    b_total: float
    delta_p: float
    delta_kv: float
    bound_p: float
    bound_kv: float
    bound_both: float
    n_star: float
    n_star_budget: float  # crossover of a KV method keeping a fixed r_kv * n tokens
    gap_per_k: float      # s (seconds per 1K tokens) at bw_eff; NaN without one
    n_lat: float          # latency crossing n* - (c_P - c_KV)/s (tokens); NaN without bw_eff


def account(dm: Dims, n_layers: int, n: float, r_p: float, r_kv: float,
            s_w: float = 2.0, s_kv: float = 2.0, proj_set: str = "all7",
            fixed_bytes: float = 0.0, bw_eff: float = 0.0, c_p: float = 0.0,
            c_kv: float = 0.0) -> Record:
    tot = b_total(dm, n_layers, n, s_w, s_kv, fixed_bytes)
    dp = delta_p(dm, n_layers, r_p, s_w, proj_set)
    dk = delta_kv(dm, n_layers, n, r_kv, s_kv)
    n_star = crossover(dm, r_p, r_kv, s_w, s_kv, proj_set) if r_kv < 1.0 else float("inf")
    nan = float("nan")
    s = gap_growth_per_k(dm, n_layers, r_kv, s_kv, bw_eff) if bw_eff > 0 else nan
    if bw_eff > 0 and r_kv < 1.0:
        n_lat = latency_crossing(n_star, c_p, c_kv, s)
    elif bw_eff > 0:
        n_lat = float("inf")
    else:
        n_lat = nan
    return Record(
        b_attn=b_attn(dm, s_w), b_mlp=b_mlp(dm, s_w), b_kv=b_kv(dm, n, s_kv),
        b_total=tot, delta_p=dp, delta_kv=dk,
        bound_p=speedup_bound(tot, dp), bound_kv=speedup_bound(tot, dk),
        bound_both=speedup_bound(tot, dp + dk), n_star=n_star,
        n_star_budget=crossover_fixed_budget(dm, r_kv * n, r_p, s_w, s_kv, proj_set),
        gap_per_k=s, n_lat=n_lat,
    )


def step_bytes(dm: Dims, n_layers: int, n_read: int, n_kept: int,
               s_w: float, s_kv: float, has_sel: bool) -> float:
    """Algorithmic HBM bytes of one decode step as this build executes it.

    Per layer: W_qkv and W_o once, W_gate densely, up and down rows of the
    n_kept kept channels (n_kept = d_ff when dense), n_read cached rows of K
    and V, and the appended key/value row written to the full cache and, when
    the layer holds a gathered buffer, to that buffer too, in every mode
    ([Cross] §3.2: nothing is discarded, the full cache keeps receiving
    entries, and the mode may change from one step to the next).  Activations, norm vectors and split-K
    partials are excluded (they are < 0.1% at the 8B-class shapes).
    """
    d, dh = dm.d_model, dm.head_dim
    qkv_out = dm.n_q_heads * dh + 2 * dm.n_kv_heads * dh
    w = s_w * (d * qkv_out + dm.n_q_heads * dh * d + d * dm.d_ff + 2 * d * n_kept)
    kv_row = 2 * dm.n_kv_heads * dh * s_kv
    appends = kv_row * (2 if has_sel else 1)
    return n_layers * (w + kv_row * n_read + appends)
