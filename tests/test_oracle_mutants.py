"""Planted mistakes in copies of the oracle sources must fail a pin.

Each mutant edits one or two expressions of a copy of the C sources in a
temporary directory, builds it with gcc and runs the pins against it.  The real
sources are never touched.  A mutant that no pin catches fails this test.
"""
import os
import shutil

import pytest

import oracle
import oracle_pins as P
import grad_pins as GP
import decode_pins as DP
import bias_pins as BP

ORACLE = "attention_oracle.c"
BLOCKED = "blocked_reference.c"
GRAD = "attention_grad_oracle.c"

# (id, file, [(original, replacement), ...])
MUTANTS = [
    ("causal_strict", ORACLE, [("J->causal ? i + 1 + (Nk - N) : Nk", "J->causal ? i + (Nk - N) : Nk")]),
    ("causal_leak", ORACLE, [("J->causal ? i + 1 + (Nk - N) : Nk", "J->causal ? i + 2 + (Nk - N) : Nk")]),
    ("cache_offset_dropped", ORACLE, [("J->causal ? i + 1 + (Nk - N) : Nk", "J->causal ? i + 1 : Nk")]),
    ("gqa_modulo", ORACLE, [("const int64_t hk = h / group;", "const int64_t hk = h % J->Hkv;")]),
    ("exp_sign", ORACLE, [("exp(s[j] - m);", "exp(m - s[j]);")]),
    ("no_scale", ORACLE, [("s[j] = J->scale * acc;", "s[j] = acc;")]),
    ("no_normalise", ORACLE, [("s[j] = l > 0.0 ? s[j] / l : 0.0;", "s[j] = s[j];")]),
    ("drop_first_value", ORACLE, [("for (int64_t j = 0; j < jend; ++j) {\n                const double *vj",
                                   "for (int64_t j = 1; j < jend; ++j) {\n                const double *vj")]),
    ("value_row_i", ORACLE, [("const double *vj = vh + j * d;", "const double *vj = vh + i * d;")]),
    ("transposed_scores", ORACLE, [("const double *qi = qh + i * d;", "const double *qi = kh + i * d;"),
                                   ("const double *kj = kh + j * d;", "const double *kj = qh + j * d;")]),
    ("lse_without_max", ORACLE, [("? m + log(l) :", "? log(l) :")]),
    ("dot_skips_last", ORACLE, [("for (int64_t t = 0; t < d; ++t)\n                acc += qi[t] * kj[t];",
                                 "for (int64_t t = 0; t + 1 < d; ++t)\n                acc += qi[t] * kj[t];")]),
    ("key_head_not_query_head", ORACLE, [("const double *kh = J->k + (b * J->Hkv + hk) * Nk * d;",
                                          "const double *kh = J->k + (b * J->Hkv + h % J->Hkv) * Nk * d;")]),
    ("blocked_no_rescale_l", BLOCKED, [("l[i] = a_old * l[i] + a_blk * lt;", "l[i] = l[i] + a_blk * lt;")]),
    ("blocked_no_rescale_o", BLOCKED, [("acc[i * d + t] = a_old * acc[i * d + t] + a_blk * pv[t];",
                                        "acc[i * d + t] = acc[i * d + t] + a_blk * pv[t];")]),
    ("blocked_alpha_sign", BLOCKED, [("const double a_old = exp(m[i] - mn);", "const double a_old = exp(mn - m[i]);")]),
    ("blocked_causal_strict", BLOCKED, [("causal ? ((i + 1 < j1) ? i + 1 : j1) : j1", "causal ? ((i < j1) ? i : j1) : j1")]),
    ("blocked_local_max_ignored", BLOCKED, [("const double p = exp(sblk[j - j0] - mt);",
                                             "const double p = exp(sblk[j - j0] - mn_unused);"),
                                            ("double lt = 0.0;", "double lt = 0.0; const double mn_unused = (m[i] > mt) ? m[i] : mt;")]),
    ("bias_ignored", ORACLE, [("s[j] += brow[j];", "s[j] += 0.0 * brow[j];")]),
    ("bias_scaled", ORACLE, [("s[j] += brow[j];", "s[j] += J->scale * brow[j];")]),
    ("bias_row_shift", ORACLE, [("+ i * J->si : NULL;", "+ (i > 0 ? i - 1 : 0) * J->si : NULL;")]),
    ("bias_head_stride_ignored", ORACLE, [("h * J->sh", "0 * J->sh")]),
    ("masked_row_lse_zero", ORACLE, [("l > 0.0 ? m + log(l) : -INFINITY", "l > 0.0 ? m + log(l) : 0.0")]),
    ("grad_no_row_term", GRAD, [("const double ds = p[j] * (dp[j] - pdp);", "const double ds = p[j] * dp[j];")]),
    ("grad_dk_unscaled", GRAD, [("dkh[j * d + t] += J->scale * ds * qi[t];", "dkh[j * d + t] += ds * qi[t];")]),
    ("grad_dq_from_v", GRAD, [("dqi[t] += J->scale * ds * kh[j * d + t];", "dqi[t] += J->scale * ds * vh[j * d + t];")]),
    ("grad_dv_uses_ds", GRAD, [("dvh[j * d + t] += p[j] * gi[t];", "dvh[j * d + t] += ds * gi[t];")]),
    ("grad_causal_strict", GRAD, [("const int64_t jend = J->causal ? i + 1 : N;", "const int64_t jend = J->causal ? i : N;")]),
    ("grad_dp_from_q", GRAD, [("acc += gi[t] * vh[j * d + t];", "acc += gi[t] * kh[j * d + t];")]),
    ("grad_gqa_first_head_only", GRAD, [("for (int64_t h = hk * G; h < (hk + 1) * G; ++h) {",
                                         "for (int64_t h = hk * G; h < hk * G + 1; ++h) {")]),
    ("grad_row_term_unweighted", GRAD, [("pdp += p[j] * acc;", "pdp += acc;")]),
]


def _quick_oracle_pins(lib):
    P.pin_brute_force(lib, quick=True)
    P.pin_torch_sdpa(lib)
    P.pin_closed_forms(lib)
    P.pin_invariants(lib)
    BP.all_bias_pins(lib)
    DP.all_decode_pins(lib)


def _quick_grad_pins(lib):
    GP.pin_grad_closed_forms(lib)
    GP.pin_grad_invariants(lib)
    GP.pin_grad_finite_differences(lib, quick=True)


def _build_mutant(tmp_path, fname, edits):
    srcs = []
    for s in oracle.SOURCES:
        dst = tmp_path / s
        shutil.copy(os.path.join(oracle.HERE, s), dst)
        srcs.append(str(dst))
    path = tmp_path / fname
    text = path.read_text()
    for old, new in edits:
        assert text.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
        text = text.replace(old, new)
    path.write_text(text)
    return oracle.load(oracle.build(str(tmp_path / "libmutant.so"), tuple(srcs)))


@pytest.mark.parametrize("mid,fname,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, mid, fname, edits):
    lib = _build_mutant(tmp_path, fname, edits)
    if fname == ORACLE:
        pins = _quick_oracle_pins
    elif fname == GRAD:
        pins = _quick_grad_pins
    else:
        pins = lambda L: P.pin_blocked_agrees(L, quick=True)
    with pytest.raises(AssertionError):
        pins(lib)
