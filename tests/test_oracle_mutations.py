"""Each plausible mistake planted in a scratch copy of the oracle must make at
least one oracle pin fail (CPU only; the repository's oracle is not touched)."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MUTS = [
 ("selection.py", "pos = n - w + np.arange(w)[:, None]", "pos = n - w + 1 + np.arange(w)[:, None]"),
 ("selection.py", "k[h // g, :n]", "k[h % k.shape[0], :n]"),
 ("selection.py", "order = np.lexsort((cand, -s))", "order = np.lexsort((-cand, -s))"),
 ("selection.py", "* scale\n    pos", "* scale * 1.01\n    pos"),
 ("attention.py", "kk = k[h // g, :n_rows]", "kk = k[h % k.shape[0], :n_rows]"),
 ("attention.py", "z = kk @ q[h].astype(np.float64) * scale\n        m = z.max()", "z = kk @ q[h].astype(np.float64)\n        m = z.max()"),
 ("attention.py", "den = (wgt * l).sum(axis=1)", "den = l.sum(axis=1)"),
 ("cats.py", "return np.abs(act_f32) > t32", "return np.abs(act_f32) >= t32"),
 ("cats.py", "return w_down_t.astype(np.float64).T @ hmid", "return w_up.astype(np.float64).T @ hmid"),
 ("cats.py", "return g / (1.0 + np.exp(-g))", "return g / (1.0 + np.exp(g))"),
 ("cats.py", "return float(v[k - 1])", "return float(v[k])"),
 ("step.py", "lo * c - hi * s, hi * c + lo * s", "lo * c + hi * s, hi * c - lo * s"),
 ("step.py", "np.sqrt(np.mean(x * x) + eps)", "np.sqrt(np.mean(x * x)) + eps"),
 ("step.py", "out[nz] = np.round(x[nz] / ulp) * ulp", "out[nz] = np.floor(x[nz] / ulp + 0.5) * ulp"),
 ("step.py", "h = h + layer.w_o @ o.reshape(-1)", "h = layer.w_o @ o.reshape(-1)"),
 ("step.py", "inv_freq = theta ** (-(2.0 * np.arange(half)) / d_h)", "inv_freq = theta ** (-(np.arange(half)) / d_h)"),
 ("byte_account.py", "return 2 * dm.d_model * dm.d_ff", "return 3 * dm.d_model * dm.d_ff"),
 ("byte_account.py", "return dm.d_model * qkv_out + dm.n_q_heads * dm.head_dim * dm.d_model", "return dm.d_model * qkv_out"),
 ("byte_account.py", "den = 2.0 * batch * dm.n_kv_heads", "den = 2.0 * dm.n_kv_heads"),
 ("teal.py", "return np.abs(x_f32) > t32", "return np.abs(x_f32) >= t32"),
 ("teal.py", "g = linear_masked(layer.w_gate, x2, m_m)", "g = linear_masked(layer.w_gate, x, m_m)"),
 ("teal.py", "m_d = mask_of(DOWN_IN, hmid)", "m_d = mask_of(DOWN_IN, u)"),
 ("teal.py", "h = h + linear_masked(layer.w_o, o, m_o)", "h = h + linear_masked(layer.w_o, o, m_a)"),
 ("teal.py", "hmid = cats.silu(g) * u", "hmid = g * u"),
 ("attention.py", "int(n_heads[kv])", "int(n_heads[0])"),
 ("step.py", "layer.k_sel[kv, layer.n_sel_heads[kv]] = k_r[kv]", "layer.k_sel[kv, layer.n_sel_heads[0]] = k_r[kv]"),
 ("selection.py", "return [min(n, int(np.floor(eta * n))) if a else min(n, int(budget)) for a in adaptive]",
  "return [min(n, int(np.floor(eta * n))) if not a else min(n, int(budget)) for a in adaptive]"),
 ("batch.py", "return np.any(m, axis=0)", "return np.all(m, axis=0)"),
 ("batch.py", "return 1.0 - (1.0 - keep) ** batch", "return 1.0 - keep ** batch"),
 ("batch.py", "for b, (layers, h, pos) in enumerate(zip(seq_layers, hs, positions)):",
  "for b, (layers, h, pos) in enumerate(zip(seq_layers, hs, positions[::-1])):"),
 ("byte_account.py", "b_kv(dm, K_TOKENS, s_kv) * (1.0 - r_kv) / bw_bytes_per_s",
  "b_kv(dm, K_TOKENS, s_kv) / bw_bytes_per_s"),
 ("selection.py", "return [cache[kv, idx] for kv, idx in enumerate(idx_list)]",
  "return [cache[0, idx] for kv, idx in enumerate(idx_list)]"),
 ("byte_account.py", "    return sbb / sbt\n", "    return sbb / sbt * len(b) / (len(b) - 1)\n"),
 ("byte_account.py", "float(t) - float(b) / bw_eff", "float(t) + float(b) / bw_eff"),
 ("byte_account.py", "* dlt[i] / (dlt[i] - dlt[i + 1])", "* dlt[i + 1] / (dlt[i] - dlt[i + 1])"),
 ("byte_account.py", "tot = horizon * float(ts) + float(to)", "tot = horizon * float(ts)"),
 ("byte_account.py", "n_star_budget=crossover_fixed_budget(dm, r_kv * n,",
  "n_star_budget=crossover_fixed_budget(dm, n,"),
]

PIN_FILES = ["tests/test_oracle_byte_account.py", "tests/test_oracle_selection.py",
             "tests/test_oracle_attention.py", "tests/test_oracle_cats.py",
             "tests/test_oracle_step.py", "tests/test_oracle_teal.py",
             "tests/test_oracle_batch.py"]


@pytest.mark.parametrize("fname,old,new", MUTS, ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTS)])
def test_planted_mistake_is_caught(tmp_path, fname, old, new):
    for sub in ("oracle", "tests", "synth"):
        shutil.copytree(os.path.join(ROOT, sub), tmp_path / sub,
                        ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp_path)
    p = tmp_path / "oracle" / fname
    s = p.read_text()
    assert old in s, "mutation site vanished from the oracle"
    p.write_text(s.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider"]
                       + PIN_FILES, cwd=tmp_path, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, "planted mistake survived every pin:\n" + r.stdout[-2000:]
