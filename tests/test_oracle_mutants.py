"""Test power of the oracle pins: plant one mistake at a time in the oracle
source (on the CPU), rebuild it, and require that some pin fails.

The battery imitates the mutation record of the LocalAI QSA-block commit
(section "The battery"): every mutant is proved applied (its edit must match
exactly once), every build's return code is checked before any pin runs, and
no mutant may survive.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as ob
import oracle_pins

SRC = ob.SRC
HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

MUTANTS = {
    "pool_divisor": ("pooled[j * d_idx + x] = acc / (float)r;",
                     "pooled[j * d_idx + x] = acc / (float)(r - 1);"),
    "pool_drops_first_token": ("for (int32_t s = 0; s < r; ++s) acc",
                               "for (int32_t s = 1; s < r; ++s) acc"),
    "score_no_relu": ("a = (a > 0.0f) ? a : 0.0f;", "a = (a > 0.0f) ? a : a;"),
    "score_no_scale": ("float a = c * d;", "float a = d;"),
    "score_weight_index": ("s = fmaf(w[h], a, s);", "s = fmaf(w[0], a, s);"),
    "score_wrong_head_query": ("const float* qh = qI + (int64_t)h * d_idx;",
                               "const float* qh = qI + (int64_t)0 * d_idx;"),
    "score_transposed_pooled": ("const float* kb = pooled + j * d_idx;",
                                "const float* kb = pooled + j;"),
    "topk_tiebreak_highest": ("return (a->j < b->j) ? -1 : (a->j > b->j);",
                              "return (a->j > b->j) ? -1 : (a->j < b->j);"),
    "topk_bottom_k": ("if (a->s > b->s) return -1;", "if (a->s < b->s) return -1;"),
    "topk_skips_best": ("sel[i] = all[i].j;", "sel[i] = all[i + 1].j;"),
    "candidates_short_by_one": ("const int64_t nb = n / r;", "const int64_t nb = (n - 1) / r;"),
    "tail_dropped_last": ("for (int64_t t = nb * r; t < n; ++t) tokens[c++] = t;",
                          "for (int64_t t = nb * r; t < n - 1; ++t) tokens[c++] = t;"),
    "tail_reads_future": ("int64_t n = p + 1, c = 0;", "int64_t n = p + 2, c = 0;"),
    "gqa_map_modulo": ("int32_t kvh = h / g;", "int32_t kvh = h % Hkv;"),
    "gate_silu": ("double gt = gate ? 1.0 / (1.0 + exp(-(double)gate[(int64_t)h * D + x])) : 1.0;",
                  "double gt = gate ? (double)gate[(int64_t)h * D + x] / (1.0 + exp(-(double)gate[(int64_t)h * D + x])) : 1.0;"),
    "attn_no_scale": ("z[i] = scale * acc;", "z[i] = acc;"),
    "pv_reads_keys": ("const float* vr = V + (tokens[i] * Hkv + kvh) * D;",
                      "const float* vr = K + (tokens[i] * Hkv + kvh) * D;"),
    "dense_layer_drops_self": ("for (int64_t t = 0; t < n; ++t) tokens[c++] = t;",
                               "for (int64_t t = 0; t + 1 < n; ++t) tokens[c++] = t;"),
    # 8-bit K/V storage and the rotated basis
    "fwht_wrong_sign": ("x[j + len] = a - b;", "x[j + len] = b - a;"),
    "e4m3_exponent_bias": ("ldexpf((float)(8 + m), e - 10)", "ldexpf((float)(8 + m), e - 9)"),
    "e4m3_ties_to_odd": ("(dn == up && ((c - 1) & 1) == 0)", "(dn == up && ((c - 1) & 1) == 1)"),
    "e4m3_no_saturation": ("if (a >= 448.0f) return sgn | 0x7E;",
                           "if (a >= 480.0f) return sgn | 0x7F;"),
    "kv8_encode_skips_rotation": ("if (rotate) qsa_oracle_fwht(t, D);",
                                  "if (0) qsa_oracle_fwht(t, D);"),
    "kv8_query_not_rotated": ("for (int64_t i = 0; i < nq * Hq; ++i) qsa_oracle_fwht(qr + i * D, D);",
                              "for (int64_t i = 0; i < 0; ++i) qsa_oracle_fwht(qr + i * D, D);"),
    "kv8_scores_not_divided": ("d2.attn_scale = (float)(a_scale / (double)D);",
                               "d2.attn_scale = (float)a_scale;"),
    "kv8_output_not_unrotated": ("        qsa_oracle_fwht(o, D);\n        for (int32_t x = 0; x < D; ++x) o[x] = o[x] / (float)D;",
                                 "        for (int32_t x = 0; x < D; ++x) o[x] = o[x] / (float)D;"),
    "kv8_v_scale_from_k": ("Vd[i] = qsa_oracle_e4m3_decode(Vc[i]) * v_scale;",
                           "Vd[i] = qsa_oracle_e4m3_decode(Vc[i]) * k_scale;"),
    "rope_sign": ("x[i] = a * c - b * sn;", "x[i] = a * c + b * sn;"),
    "rope_second_half_sign": ("x[i + h] = b * c + a * sn;", "x[i + h] = b * c - a * sn;"),
    "rope_frequency_exponent": ("pow(theta, -2.0 * (double)i / (double)R)",
                                "pow(theta, -1.0 * (double)i / (double)R)"),
    "rope_adjacent_pairs": ("const float a = x[i], b = x[i + h];",
                            "const float a = x[i], b = x[i ^ 1];"),
    "pooled_rope_block_index": ("(double)dm->idx_rope_theta, j * r);",
                                "(double)dm->idx_rope_theta, j);"),
    "pooled_rope_skipped": ("if (dm->idx_rope_dim > 0)\n", "if (dm->idx_rope_dim > 100000)\n"),
}

# Mistakes planted in the block front end (oracle/block.py), one at a time.
PY_SRC = os.path.join(ROOT, "oracle", "block.py")
PY_MUTANTS = {
    "norm_weight_polarity": ("* (1.0 + widen(w).astype(np.float64))",
                             "* (widen(w).astype(np.float64))"),
    "norm_sum_not_mean": ("ms = np.mean(x64 * x64, axis=-1, keepdims=True)",
                          "ms = np.sum(x64 * x64, axis=-1, keepdims=True)"),
    "gate_rows_before_q": ('sizes = [("q", Hq * D), ("gate", Hq * D),',
                           'sizes = [("gate", Hq * D), ("q", Hq * D),'),
    "query_rope_next_position": ('t = orc.rope(t, bd["rotary_dim"], bd["rope_theta"], pos[:, None])',
                                 't = orc.rope(t, bd["rotary_dim"], bd["rope_theta"], pos[:, None] + 1)'),
    "index_query_not_rotated": ('t = orc.rope(P.reshape(n, HI, dI), bd["idx_rope_dim"],',
                                't = orc.rope(P.reshape(n, HI, dI), 0,'),
    "k_norm_uses_q_weight": ('qn_w if name == "q" else kn_w', 'qn_w'),
    "o_proj_of_unrounded": ('ref["y"] = project(attn, W_o)', 'ref["y"] = project(attn * 1.01, W_o)'),
}


def test_every_mutant_is_distinct_and_applies():
    text = open(SRC).read()
    for name, (a, b) in MUTANTS.items():
        assert text.count(a) == 1, name
        assert a != b, name
    text = open(PY_SRC).read()
    for name, (a, b) in PY_MUTANTS.items():
        assert text.count(a) == 1, name
        assert a != b, name


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_killed(name, tmp_path):
    a, b = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(a) == 1
    src = tmp_path / "mut.c"
    src.write_text(text.replace(a, b))
    lib = str(tmp_path / "libmut.so")
    ob.build(lib, str(src))                 # raises if the build fails
    assert os.path.exists(lib)
    # Each mutant runs in a child process: a mutant that corrupts memory and
    # aborts is killed too, and cannot take the test session down with it.
    code = (
        "import sys, oracle, oracle_pins\n"
        f"m = oracle.load({lib!r})\n"
        "failed = []\n"
        "for pin in oracle_pins.ALL_PINS:\n"
        "    try:\n"
        "        pin(m)\n"
        "    except (AssertionError, ValueError):\n"
        "        failed.append(pin.__name__)\n"
        "print('FAILED_PINS', failed)\n"
        "sys.exit(1 if failed else 0)\n")
    env = dict(os.environ)
    env["PYTHONPATH"] = os.pathsep.join([ROOT, HERE, env.get("PYTHONPATH", "")])
    env["OMP_NUM_THREADS"] = "2"
    proc = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                          text=True, timeout=300)
    assert proc.returncode != 0, f"mutant {name} survived every pin"


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_block_mutant_is_killed(name, tmp_path):
    """A copy of the oracle package with one mistake in block.py, loaded
    first on the path of a child process, against the unmodified C oracle."""
    import shutil
    a, b = PY_MUTANTS[name]
    text = open(PY_SRC).read()
    assert text.count(a) == 1
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    for f in ("__init__.py", "build.py"):
        shutil.copy(os.path.join(ROOT, "oracle", f), pkg / f)
    (pkg / "block.py").write_text(text.replace(a, b))
    lib = os.path.join(ROOT, "oracle", "libqsa_oracle.so")
    if not os.path.exists(lib):
        ob.build(lib)
    code = (
        "import sys, oracle, oracle_pins\n"
        "assert oracle.__file__.startswith(%r)\n"
        f"m = oracle.load({lib!r})\n"
        "failed = []\n"
        "for pin in oracle_pins.ALL_PINS:\n"
        "    try:\n"
        "        pin(m)\n"
        "    except (AssertionError, ValueError):\n"
        "        failed.append(pin.__name__)\n"
        "print('FAILED_PINS', failed)\n"
        "sys.exit(1 if failed else 0)\n") % str(tmp_path)
    env = dict(os.environ)
    env["PYTHONPATH"] = os.pathsep.join([str(tmp_path), ROOT, HERE, env.get("PYTHONPATH", "")])
    env["OMP_NUM_THREADS"] = "2"
    proc = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                          text=True, timeout=300, cwd=str(tmp_path))
    assert "FAILED_PINS" in proc.stdout, proc.stderr[-2000:]
    assert proc.returncode != 0, f"mutant {name} survived every pin"
