"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a private copy of the oracle's C source, builds
it, and runs the pin suite against it in a subprocess; the suite must fail.
Nothing here touches the GPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fa_oracle.c")

# (name, text in fa_oracle.c, planted replacement)
MUTANTS = [
    ("gqa_map_modulo", "const int64_t n2 = n1 / (p->QN / p->KVN);\n    double m",
     "const int64_t n2 = n1 % p->KVN;\n    double m"),
    ("scale_dropped", "s[j] = p->scale * acc;", "s[j] = acc;"),
    ("causal_off_by_one", "if (p->mask_mode == 1 && j > i) return 0;",
     "if (p->mask_mode == 1 && j >= i) return 0;"),
    ("lse_base2", "jb->lse[r] = log(l) + m;", "jb->lse[r] = log2(l) + m;"),
    ("length_ignored", "int64_t L = p->lens ? p->lens[b] : cap;", "int64_t L = cap;"),
    ("mask_polarity", "if (p->mask[b * st[0] + n1 * st[1] + i * st[2] + j * st[3]] != 0) return 0;",
     "if (p->mask[b * st[0] + n1 * st[1] + i * st[2] + j * st[3]] == 0) return 0;"),
    ("merge_weight_sign", "const double w = exp(m[c] - mg);", "const double w = exp(mg - m[c]);"),
    ("partial_normalised",
     "jb->l_part[r * jb->splits + c] = weighted_values(p, jb->v, b, n1, j0, j1, s, ok, m, o);",
     "jb->l_part[r * jb->splits + c] = weighted_values(p, jb->v, b, n1, j0, j1, s, ok, m, o);"
     " for (int64_t d = 0; d < p->D; ++d) o[d] /= jb->l_part[r * jb->splits + c];"),
    ("value_row_offset", "const uint16_t *vr = v + kv_index(p, b, n2, j);",
     "const uint16_t *vr = v + kv_index(p, b, n2, j > 0 ? j - 1 : 0);"),
    ("bf16_decode_shift", "uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    ("window_left_bound", "if (p->win_left >= 0 && j < i - p->win_left) return 0;",
     "if (p->win_left >= 0 && j <= i - p->win_left) return 0;"),
    ("window_right_sign", "if (p->win_right >= 0 && j > i + p->win_right) return 0;",
     "if (p->win_right >= 0 && j > i - p->win_right) return 0;"),
    ("tnd_kv_offsets", "if (p->layout == 2) return ((p->cu_kv[b] + j) * p->KVN + n) * p->D;",
     "if (p->layout == 2) return ((p->cu_q[b] + j) * p->KVN + n) * p->D;"),
    ("tnd_used_rows", "(p->used_q && i >= p->used_q[b]))", "(p->used_q && i > p->used_q[b]))"),
    ("padded_used_rows", "if (p->used_q && i >= p->used_q[b]) computed = 0;",
     "if (p->used_q && i > p->used_q[b]) computed = 0;"),
    ("paged_row_offset", "const int64_t r = j % p->block_size;", "const int64_t r = (j + 1) % p->block_size;"),
    ("paged_bnbd_order", ": ((blk * p->KVN + n) * p->block_size + r) * p->D;",
     ": ((blk * p->block_size + r) * p->KVN + n) * p->D;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread", "-o",
                           str(lib), str(mutant), "-lm"])
    env = dict(os.environ, FA_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
