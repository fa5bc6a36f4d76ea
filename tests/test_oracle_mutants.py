"""The oracle's pins must fail on plausible mistakes.

Each case plants one mistake in a copy of the oracle source (on the CPU), builds it, and
runs the pin suite against that copy in a subprocess: the suite must fail.  Nothing here
touches the GPU or the real oracle build.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTANTS = {
    # routing
    "ties_to_higher_index": ("(ka == kb && a < b)", "(ka == kb && a > b)"),
    "weights_not_renormalised": ("renormalize ? val[sel[j]] / norm : val[sel[j]]", "val[sel[j]]"),
    "bias_in_weight": ("val[e] = s[e];", "val[e] = key[e];"),
    "group_score_top1_only": ("key[top[0]] + key[top[1]] : key[top[0]]", "key[top[0]] : key[top[0]]"),
    "sigmoid_in_fp32": ("(float)(1.0 / (1.0 + exp(-(double)x)))", "1.0f / (1.0f + expf(-x))"),
    # align
    "align_unpadded": ("total += (expert_counts[e] + BM - 1) / BM * BM;", "total += expert_counts[e];"),
    "align_reverse_within_expert": ("for (int64_t i = 0; i < pairs; i++) {\n        int64_t r = next",
                                    "for (int64_t i = pairs - 1; i >= 0; i--) {\n        int64_t r = next"),
    # FFN
    "gate_up_swapped": ("h[i] = silu(g) * u;", "h[i] = silu(u) * g;"),
    "last_slot_dropped": ("for (int j = 0; j < k; j++) {\n            int e = jb->ids",
                          "for (int j = 0; j < k - 1; j++) {\n            int e = jb->ids"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "int4_nibbles_swapped": ("(c % 2 == 0) ? (byte & 0xF) : (byte >> 4)", "(c % 2 == 0) ? (byte >> 4) : (byte & 0xF)"),
    "int4_zero_ignored": ("return ((double)q - z) * s;", "return (double)q * s;"),
    "int4_group_64": ("(cols / 128) + c / 128) * rows + n;", "(cols / 128) + c / 256) * rows + n;"),
    "int4_scales_row_major": ("(cols / 128) + c / 128) * rows + n;", "rows + n) * (cols / 128) + c / 128;"),
    "int4_row_nibbles_swapped": ("(c % 2 == 0) ? (row[c / 2] & 0xF) : (row[c / 2] >> 4)",
                                 "(c % 2 == 0) ? (row[c / 2] >> 4) : (row[c / 2] & 0xF)"),
    "int4_row_zero_ignored": ("buf[c] = ((double)q - z) * s;", "buf[c] = (double)q * s;"),
    "bf16_row_transposed": ("((int64_t)e * rows + n) * cols;\n        for (int64_t c = 0; c < cols; c++) buf[c] = orc_bf16_to_f32(row[c]);",
                            "((int64_t)e * rows) * cols + n;\n        for (int64_t c = 0; c < cols; c++) buf[c] = orc_bf16_to_f32(row[c * rows]);"),
    "fp8_row_scale_of_other_matrix": ("double scale = (m == 0 ? W->w13_scale : W->w2_scale)[e];",
                                      "double scale = W->w13_scale[e];"),
    # fp8 and codecs
    "e4m3_ties_to_odd": ("((lo & 1) ? hi : lo)", "((lo & 1) ? lo : hi)"),
    "e4m3_bias_8": ("ex - 7);\n    return (float)(sign ? -v : v);\n}\n\n/* Round",
                    "ex - 8);\n    return (float)(sign ? -v : v);\n}\n\n/* Round"),
    "a2_scale_from_a1": ("pertensor_scales(amax2, &s2, &inv2);", "pertensor_scales(amax1, &s2, &inv2);"),
    # grouped GEMM
    "ggemm_scale_of_next_expert": ("(double)x_scale * w_scale[e] : 1.0;", "(double)x_scale * w_scale[(e + 1) % E] : 1.0;"),
    "ggemm_weight_transposed": ("grouped_elem(dtype, w, wrow + c)", "grouped_elem(dtype, w, (int64_t)e * N * K + (int64_t)c * N + n)"),
    "ggemm_segments_from_zero": ("for (int i = 0; i < m_sizes[e]; i++, r++) {", "for (int i = 0; i < m_sizes[e]; i++, r++) { r = r % (m_sizes[e] ? m_sizes[e] : 1);"),
    "bf16_truncates": ("if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;", ""),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not found: " + name
    mut = tmp_path / "moe_oracle.c"
    mut.write_text(src.replace(old, new))
    (tmp_path / "moe_oracle.h").write_text(open(os.path.join(ROOT, "oracle", "moe_oracle.h")).read())
    so = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-pthread", "-fPIC", "-shared", str(mut), "-lm", "-o", str(so)])
    env = dict(os.environ, MOE_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "pins did not catch mutant " + name
