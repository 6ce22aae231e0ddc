"""Mutation test of the pins: plausible mistakes planted in a copy of the
oracle's C source (on the CPU) must each make at least one pin fail."""
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attn_oracle.c")

# (name, original text, mutated text)
MUTANTS = [
    ("causal_off_by_one", "return (i + 1 < n_k) ? i + 1 : n_k;", "return (i < n_k) ? i : n_k;"),
    ("causal_ignored", "if (!causal) return n_k;", "return n_k;"),
    ("scale_dropped", "s[j - j0] = scale * dot;", "s[j - j0] = dot;"),
    ("scale_squared", "s[j - j0] = scale * dot;", "s[j - j0] = scale * scale * dot;"),
    ("max_not_subtracted_in_lse", "*lse = m + log(l);", "*lse = log(l);"),
    ("values_from_keys", "const double* vj = V + j * d;", "const double* vj = K + j * d;"),
    ("normalisation_dropped", "for (int c = 0; c < d; ++c) o[c] /= l;", ""),
    ("log2_lse", "*lse = m + log(l);", "*lse = m + log2(l);"),
    ("merge_weights_dropped", "const double w = exp(mc - M);", "const double w = 1.0;"),
    ("feature_index_reversed", "for (int c = 0; c < d; ++c) dot += q[c] * kj[c];",
     "for (int c = 0; c < d; ++c) dot += q[c] * kj[d - 1 - c];"),
    ("window_left_off_by_one", "if (wl >= 0 && i - wl > lo) lo = i - wl;", "if (wl >= 0 && i - wl + 1 > lo) lo = i - wl + 1;"),
    ("window_right_off_by_one", "if (wr >= 0 && i + wr + 1 < hi) hi = i + wr + 1;", "if (wr >= 0 && i + wr < hi) hi = i + wr;"),
    ("window_sides_swapped", "if (wl >= 0 && i - wl > lo) lo = i - wl;", "if (wr >= 0 && i - wr > lo) lo = i - wr;"),
    ("window_empty_lse_zero", "*lse = -INFINITY; /* o is already zero */", "*lse = 0.0;"),
    ("bwd_ds_sign", "dS[i * n_k + j] = prow[j] * (dp - Di);", "dS[i * n_k + j] = prow[j] * (dp + Di);"),
    ("bwd_dq_scale_dropped", "gq[i * d + c] = scale * acc;", "gq[i * d + c] = acc;"),
    ("bwd_dk_from_p", "acck += dS[i * n_k + j] * q[i * d + c];", "acck += P[i * n_k + j] * q[i * d + c];"),
    ("bwd_dv_from_ds", "accv += P[i * n_k + j] * go[i * d + c];", "accv += dS[i * n_k + j] * go[i * d + c];"),
    ("bwd_D_from_v", "Di += go[i * d + c] * oc;", "Di += go[i * d + c] * v[c];"),
    ("bwd_causal_ignored", "const int64_t n_allowed = allowed_prefix(i, n_k, causal);\n      double* prow = P + i * n_k;",
     "const int64_t n_allowed = allowed_prefix(i, n_k, 0);\n      double* prow = P + i * n_k;"),
    ("e4m3_bias_8", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    ("e4m3_subnormal_scale", "ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    ("e4m3_ties_away", "if (r > 0.5 || (r == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;", "if (r >= 0.5) fl += 1.0;"),
    ("e4m3_truncate", "if (r > 0.5 || (r == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;", ""),
    ("quant_range_240", "const float inv = amax > 0.f ? 448.0f / amax : 1.0f;",
     "const float inv = amax > 0.f ? 240.0f / amax : 1.0f;"),
    ("quant_descale_inverted", "descale[bh] = amax > 0.f ? amax / 448.0f : 1.0f;",
     "descale[bh] = amax > 0.f ? 448.0f / amax : 1.0f;"),
    ("fp8_v_descale_from_k", "Vh[e] = table[vc[e]] * (double)descale_v[bh];", "Vh[e] = table[vc[e]] * (double)descale_k[bh];"),
    ("fp8_q_descale_head0", "q[c] = table[Qc[rows[r] * d + c]] * (double)descale_q[bh];",
     "q[c] = table[Qc[rows[r] * d + c]] * (double)descale_q[0];"),
    ("blockmask_key_block_by_query", "return mrow[j / bk] != 0;", "return mrow[i / bk] != 0;"),
    ("blockmask_head_from_batch", "return M + (((b % Mb) * Mh + (h % Mh)) * n_qb + i / bq) * n_kb;",
     "return M + (((b % Mb) * Mh + (b % Mh)) * n_qb + i / bq) * n_kb;"),
    ("blockmask_query_block_ignored", "return M + (((b % Mb) * Mh + (h % Mh)) * n_qb + i / bq) * n_kb;",
     "return M + (((b % Mb) * Mh + (h % Mh)) * n_qb + 0) * n_kb;"),
    ("blockmask_band_left_ignored", "  if (wl >= 0 && j < i - wl) return 0;\n  if (wr >= 0 && j > i + wr) return 0;",
     "  if (wr >= 0 && j > i + wr) return 0;"),
    ("blockmask_empty_lse_zero", "*lse = -INFINITY; /* no visible key: O stays zero */", "*lse = 0.0;"),
    ("first_key_skipped", "for (int64_t j = j0; j < j1; ++j) {\n    double p = exp", "for (int64_t j = j0 + 1; j < j1; ++j) {\n    double p = exp"),
]


def _build_mutant(tmp_path, name, before, after):
    text = open(SRC).read()
    assert before in text, f"mutation site for {name} not found"
    pkg = tmp_path / f"oracle_mut_{name}"
    shutil.copytree(os.path.join(ROOT, "oracle"), pkg,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__", "*.tmp"))
    (pkg / "attn_oracle.c").write_text(text.replace(before, after, 1))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(pkg / "liboracle.so"),
                    str(pkg / "attn_oracle.c"), "-lm"], check=True)
    spec = importlib.util.spec_from_file_location(pkg.name, pkg / "__init__.py",
                                                  submodule_search_locations=[str(pkg)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[pkg.name] = mod
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,before,after", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, before, after):
    mod = _build_mutant(tmp_path, name, before, after)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
