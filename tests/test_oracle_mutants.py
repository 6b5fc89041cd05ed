"""The oracle's pins must catch plausible mistakes (no GPU).

Each case copies the C oracle, plants one mistake by a textual edit (a dropped term, a wrong sign, an
off-by-one exponent, a transposed operand, a swapped rotation angle), builds the copy into a temporary
library, and checks that the pin tests fail against it. The mistakes live only in these temporary copies.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "retention_oracle.c")

MUTANTS = {
    "xi_off_by_one": ("pow(g, (double)(j + 1))", "pow(g, (double)(j))"),
    "zeta_off_by_one": ("pow(g, (double)(L - 1 - l))", "pow(g, (double)(L - l))"),
    "carry_decay_dropped": ("R[e] = gL * R[e] + U[e]", "R[e] = R[e] + U[e]"),
    "cross_term_dropped": ("oj[c] += QR[(size_t)j * dv + c] * xi", "oj[c] += 0.0 * xi"),
    "mask_not_causal": ("(l <= j) ?", "(l < L) ?"),
    "rotation_sign": ("dst[2 * i] = x0 * c - x1 * s", "dst[2 * i] = x0 * c + x1 * s"),
    "recurrent_read_before_update": (
        "        for (int i = 0; i < dk; ++i)\n"
        "            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] = g * S[(size_t)i * dv + j] + kr[i] * vn[j];\n"
        "        double* on = out_row(J->o, N, H, dv, b, n, h);\n"
        "        for (int j = 0; j < dv; ++j) on[j] = 0.0;\n"
        "        for (int i = 0; i < dk; ++i)\n"
        "            for (int j = 0; j < dv; ++j) on[j] += qr[i] * S[(size_t)i * dv + j];\n",
        "        double* on = out_row(J->o, N, H, dv, b, n, h);\n"
        "        for (int j = 0; j < dv; ++j) on[j] = 0.0;\n"
        "        for (int i = 0; i < dk; ++i)\n"
        "            for (int j = 0; j < dv; ++j) on[j] += qr[i] * S[(size_t)i * dv + j];\n"
        "        for (int i = 0; i < dk; ++i)\n"
        "            for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] = g * S[(size_t)i * dv + j] + kr[i] * vn[j];\n"),
    "recurrent_no_decay": ("= g * S[(size_t)i * dv + j] + kr[i] * vn[j]", "= S[(size_t)i * dv + j] + kr[i] * vn[j]"),
    "parallel_decay_exponent": ("pow(gamma, (double)(n - m))", "pow(gamma, (double)(n - m + 1))"),
    "transposed_state_read": ("const double* Ri = R + (size_t)i * dv;", "const double* Ri = R + (size_t)i;"),
    "position_origin": ("theta, pos0 + n);\n        gather_plain", "theta, n);\n        gather_plain"),
    "groupnorm_unbiased_variance": ("var /= dv;", "var /= (dv - 1);"),
    "groupnorm_eps_dropped": ("const double inv = 1.0 / sqrt(var + eps);", "const double inv = 1.0 / sqrt(var);"),
    "groupnorm_mean_kept": ("double z = (o[base + c] - mean) * inv;", "double z = o[base + c] * inv;"),
    "swish_sign": ("(1.0 + exp(-g[base + c]))", "(1.0 + exp(g[base + c]))"),
    "decay_norm_without_root": ("D /= sqrt(dsum);", "D /= dsum;"),
    "score_norm_without_abs": ("den = fabs(rsum) > 1.0 ? fabs(rsum) : 1.0;", "den = rsum > 1.0 ? rsum : 1.0;"),
    "score_scale_by_dv": ("qk /= sqrt((double)dk);", "qk /= sqrt((double)dv);"),
    "grad_adjoint_no_decay": ("S[(size_t)i * dv + j] = g * S[(size_t)i * dv + j] + qn[i] * don[j];",
                              "S[(size_t)i * dv + j] = S[(size_t)i * dv + j] + qn[i] * don[j];"),
    "grad_unrotate_sign": ("d[2 * i] = c * a + s * b;", "d[2 * i] = c * a - s * b;"),
    "grad_dv_from_q": ("for (int i = 0; i < dk; ++i) acc += kn[i] * S[(size_t)i * dv + j];",
                       "for (int i = 0; i < dk; ++i) acc += qn[i] * S[(size_t)i * dv + j];"),
    "grad_dq_reads_state_transposed": ("for (int j = 0; j < dv; ++j) acc += S[(size_t)i * dv + j] * don[j];",
                                       "for (int j = 0; j < dv; ++j) acc += S[(size_t)j * dk + i] * don[j];"),
    # normalized forms carried through a state
    "norm_key_sum_no_decay": ("z[i] = g * z[i] + kr[i];", "z[i] = z[i] + kr[i];"),
    "norm_decay_row_local_index": ("norm_row_factor(J->norm, dk, g, J->pos0 + t0 + j, rs[j])",
                                   "norm_row_factor(J->norm, dk, g, t0 + j, rs[j])"),
    "norm_rowsum_cross_exponent": ("pow(g, (double)(j + 1)) * dot(", "pow(g, (double)(j)) * dot("),
    "norm_key_sum_chunk_zeta": ("pow(g, (double)(L - 1 - l)) * Kc[", "pow(g, (double)(L - l)) * Kc["),
    "norm_scores_before_scaling": ("const double r = c * qz;", "const double r = qz;"),
}

PIN_TESTS = ["test_oracle_pins.py", "test_oracle_forms.py", "test_oracle_epilogue.py", "test_oracle_grad.py",
             "test_oracle_normalized.py"]


def _run_pins_against(src_text, tmp_path):
    """Build ``src_text`` as a temporary oracle and run the pin tests against it; returns the result."""
    mutated = src_text
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    (pkg / "retention_oracle.c").write_text(mutated)
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), pkg / "__init__.py")
    subprocess.run(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-pthread", str(pkg / "retention_oracle.c"),
                    "-o", str(pkg / "liboracle.so"), "-lm"], check=True)
    tests = tmp_path / "tests"
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tests / "golden")
    for f in ["conftest.py"] + PIN_TESTS:
        shutil.copy(os.path.join(ROOT, "tests", f), tests / f)
    env = dict(os.environ)
    # the temporary tree's conftest puts it first on sys.path, so its mutated oracle shadows the real one;
    # the package with the seeded inputs still comes from the repository
    env["PYTHONPATH"] = ROOT
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "--rootdir", str(tmp_path), "-c", os.devnull] + [str(tests / f) for f in PIN_TESTS],
                       env=env, cwd=str(tmp_path), capture_output=True, text=True, timeout=600)
    return r


def test_unmutated_copy_passes(tmp_path):
    """Control: the harness itself runs the pins green on an unmodified copy."""
    r = _run_pins_against(open(SRC).read(), tmp_path)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: %s" % name
    r = _run_pins_against(src.replace(old, new, 1), tmp_path)
    assert r.returncode != 0, "planted mistake %r was not caught by the pins:\n%s" % (name, r.stdout[-2000:])
    assert "failed" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
