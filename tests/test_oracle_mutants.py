"""Planted mistakes in the oracle must fail its pins.

Each case copies oracle.c to a temporary directory, plants one plausible
mistake (a dropped term, a wrong sign or index, a transposed operand, a
missing bias, ...), builds it with gcc, and runs the pin suite
(tests/test_oracle.py) against that build in a child process.  The child must
fail; if it passes, the pins have a blind spot.  All of this runs on the CPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "drop_first_term": ("    acc += p;\n", "    if (k) acc += p;\n"),
    "alpha_sign": ("+ (double)alpha * acc;", "- (double)alpha * acc;"),
    "beta_sign": ("return (double)beta * s;", "return -(double)beta * s;"),
    "transposed_mat2": ("mat2[k * N + j]", "mat2[j * K + k]"),
    "self_broadcast_row": ("(double)self[j];", "(double)self[i % N];"),
    "beta_zero_reads_self": ("if (beta == 0.0f) return 0.0;", ""),
    "sabs_signed": ("aabs += fabs(p);", "aabs += p;"),
    "pad_sign": ("int64_t ih = oh * c->sH - c->pH + kh * c->dH;",
                 "int64_t ih = oh * c->sH + c->pH + kh * c->dH;"),
    "dilation_dropped": ("int64_t iw = ow * c->sW - c->pW + kw * c->dW;",
                         "int64_t iw = ow * c->sW - c->pW + kw;"),
    "w_stride_uses_h": ("int64_t iw = ow * c->sW", "int64_t iw = ow * c->sH"),
    "weight_kh_kw_swapped": ("* c->KH + kh) * c->KW + kw]", "* c->KH + kw) * c->KW + kh]"),
    "bias_dropped": ("(bias ? (double)bias[oc] : 0.0)", "0.0"),
    "out_size_off_by_one": ("return span / s + 1;", "return (span + 1) / s + 1;"),
    "linear_weight_k_misindexed": ("(double)w[n * K + k]", "(double)w[n * K + (K - 1 - k)]"),
    "linear_bias_dropped": ("*ref = (bias ? (double)bias[n] : 0.0) + acc;", "*ref = acc;"),
    "grouped_input_channel_ignores_group": ("int64_t ic = g * icg + icl;", "int64_t ic = icl;"),
    "grouped_weight_index": ("w[((oc * icg + icl) * c->KH", "w[((oc * icg + (icg - 1 - icl)) * c->KH"),
    "sdpa_scale_dropped": ("s[j] = (double)scale * dot + mk;", "s[j] = dot + mk;"),
    "sdpa_mask_dropped": ("double mk = mask ? (double)mask[(bh * Sq + i) * Skv + j] : 0.0;",
                          "double mk = 0.0;"),
    "sdpa_mask_transposed": ("(double)mask[(bh * Sq + i) * Skv + j]", "(double)mask[(bh * Skv + j) * Sq + i]"),
    "sdpa_keys_reversed": ("const float* kj = k + (bh * Skv + j) * D;",
                           "const float* kj = k + (bh * Skv + (Skv - 1 - j)) * D;"),
    "sdpa_not_normalised": ("o += exp(s[j] - m) / l *", "o += exp(s[j] - m) *"),
    "sdpa_value_transposed": ("* (double)v[(bh * Skv + j) * D + d];", "* (double)v[(bh * D + d) * Skv + j];"),
    "sdpa_scale_applied_after_mask": ("s[j] = (double)scale * dot + mk;", "s[j] = (double)scale * (dot + mk);"),
    "nhwc_input_read_as_nchw": ("x[((b * c->H + ih) * c->W + iw) * c->IC + ic]",
                                "x[((b * c->IC + ic) * c->H + ih) * c->W + iw]"),
    "nhwc_weight_read_as_oihw": ("w[((oc * c->KH + kh) * c->KW + kw) * c->IC + ic]",
                                 "w[((oc * c->IC + ic) * c->KH + kh) * c->KW + kw]"),
    "nhwc_output_written_as_nchw": ("int64_t o = ((b * c.OH + oh) * c.OW + ow) * OC + oc;",
                                    "int64_t o = ((b * OC + oc) * c.OH + oh) * c.OW + ow;"),
    "convt_pad_sign": ("int64_t oh = ih * sH - pH + kh * dH;", "int64_t oh = ih * sH + pH + kh * dH;"),
    "convt_weight_ic_oc_swapped": ("w[((ic * OC + oc) * KH + kh) * KW + kw]",
                                   "w[((oc * IC + ic) * KH + kh) * KW + kw]"),
    "convt_output_padding_ignored": ("d * (k - 1) + op + 1;", "d * (k - 1) + 1;"),
    "convt_gather_dilation_dropped": ("int64_t th = oh + pH - kh * dH;", "int64_t th = oh + pH - kh;"),
    "im2col_row_order": ("int64_t kk = (ic * KH + kh) * KW + kw;",
                         "int64_t kk = (ic * KW + kw) * KH + kh;"),
}


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    c_file = tmp_path / "oracle_mutant.c"
    c_file.write_text(mutated)
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(lib),
                           str(c_file), "-lm"])
    env = dict(os.environ, BAIM_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    proc = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert proc.returncode != 0, f"pins missed planted mistake {name}:\n{proc.stdout[-2000:]}"
