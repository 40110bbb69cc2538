"""Planted mistakes: each mutant is a copy of the oracle's C source with one
plausible error (a dropped term, a wrong sign, a wrong index or operand, an
off-by-one in the causal mask). The pin suite must fail on every one of them,
which shows that the pins constrain every part of the oracle.

Runs on the CPU only; the mutants are built in a temporary directory.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, original text, replacement) -- every original must occur exactly once
MUTANTS = [
    ("fwd_scale_dropped", "p[j] = scale * dot(Q + (size_t)i * d, K + (size_t)j * d, d);",
     "p[j] = dot(Q + (size_t)i * d, K + (size_t)j * d, d);"),
    ("causal_ignored", "if (vis->causal && j > i + vis->offset) return 0;", "if (0) return 0;"),
    ("causal_off_by_one", "if (vis->causal && j > i + vis->offset) return 0;",
     "if (vis->causal && j > i + vis->offset + 1) return 0;"),
    ("lse_max_dropped", "*lse_i = m + log(l);", "*lse_i = log(l);"),
    ("normalisation_dropped", "for (int j = 0; j < N; ++j) if (visible(vis, i, j)) p[j] /= l;", ""),
    ("o_uses_k", "o_i[c] += p[j] * V[(size_t)j * d + c];", "o_i[c] += p[j] * K[(size_t)j * d + c];"),
    ("score_transposed_pass2",
     "exp(scale * dot(Q + (size_t)i * d, K + (size_t)j * d, d) - lse_h[i]);",
     "exp(scale * dot(Q + (size_t)j * d, K + (size_t)i * d, d) - lse_h[i]);"),
    ("dp_transposed", "dp[j] = dot(dO + (size_t)i * d, V + (size_t)j * d, d);",
     "dp[j] = dot(dO + (size_t)j * d, V + (size_t)i * d, d);"),
    ("D_drops_p", "Dp += p[j] * dp[j];", "Dp += dp[j];"),
    ("dS_sign", "const double ds = p[j] * (dp[j] - Dp);", "const double ds = p[j] * (dp[j] + Dp);"),
    ("dq_uses_v", "dq_i[c] += ds * K[(size_t)j * d + c];", "dq_i[c] += ds * V[(size_t)j * d + c];"),
    ("dq_scale_dropped", "for (int c = 0; c < d; ++c) dq_i[c] *= scale;", ""),
    ("dk_uses_dO", "dk_j[c] += ds * Q[(size_t)i * d + c];", "dk_j[c] += ds * dO[(size_t)i * d + c];"),
    ("dk_scale_dropped", "for (int c = 0; c < d; ++c) dk_j[c] *= scale;", ""),
    ("dv_uses_q", "dv_j[c] += pij * dO[(size_t)i * d + c];", "dv_j[c] += pij * Q[(size_t)i * d + c];"),
    ("column_visibility_transposed", "if (!visible(&vis, i, j)) continue;   /*",
     "if (!visible(&vis, j, i)) continue;   /*"),
    # block-sparse attention
    ("block_index_transposed", "vis->blocks[(size_t)(i / vis->bs) * vis->nb + j / vis->bs]",
     "vis->blocks[(size_t)(j / vis->bs) * vis->nb + i / vis->bs]"),
    ("block_edge_off_by_one", "vis->nb + j / vis->bs] != 0",
     "vis->nb + (j > 0 ? j - 1 : 0) / vis->bs] != 0"),
    ("empty_row_lse_zero", "*lse_i = -INFINITY;", "*lse_i = 0.0;"),
    ("column_pass_ignores_blocks", "if (!visible(&vis, i, j)) continue;   /*",
     "if (vis.causal && j > i) continue;   /*"),
    ("head_stride_ignored", "v.blocks = mask ? mask + mask_stride * bh : NULL;", "v.blocks = mask;"),
    # queries over a key/value cache
    ("cache_offset_dropped", "vis.offset = Nk - Nq;", "vis.offset = 0;"),
    ("cache_offset_off_by_one", "vis.offset = Nk - Nq;", "vis.offset = Nk - Nq - 1;"),
    ("cache_query_head_stride", "forward_row(q + (size_t)bh * Nq * d,", "forward_row(q + (size_t)bh * Nk * d,"),
    ("dS_uses_pass1_D_minus", "const double ds = pij * (dpij - D_h[i]);", "const double ds = pij * dpij;"),
    # backward over Nq queries and Nk keys
    ("bwd_kv_offset_dropped", "Nk - Nq /* causal offset */", "0 /* causal offset */"),
    ("pass2_offset_dropped", "vis.offset = offset;   /* pass 2 */", ""),
    ("pass2_query_head_stride", "kh = (size_t)bh * Nk * d, qh = (size_t)bh * Nq * d;",
     "kh = (size_t)bh * Nk * d, qh = (size_t)bh * Nk * d;"),
    ("pass2_lse_head_stride", "lse_h = lse + (size_t)bh * Nq;", "lse_h = lse + (size_t)bh * Nk;"),
]


def test_mutants_are_well_formed():
    src = open(SRC).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) == 1, name


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, tmp_path):
    src = open(SRC).read()
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new, 1))
    lib = str(tmp_path / "liboracle_mutant.so")
    oracle.compile_c(str(mutated), lib)
    env = dict(os.environ, ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
