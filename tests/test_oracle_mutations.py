"""Planted mistakes: each mutation below is a plausible slip in the oracle
(a dropped term, a wrong comparison, a wrong index).  Every one is compiled
into a scratch copy of the oracle and the pin suite must fail against it.
Runs on the CPU only; nothing here touches the GPU library."""
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SRC = (ROOT / "oracle" / "focus_oracle.c").read_text()

MUTATIONS = {
    "window_le": ("int in_window = (i - j) < w;", "int in_window = (i - j) <= w;"),
    "same_set_not_shared": ("int shares = (bk[i] & bk[j]) != 0;",
                            "int shares = bk[i] == bk[j];"),
    "fused_score": ("float p = r[e] * c[e];\n        s = s + p;",
                    "s = fmaf(r[e], c[e], s);"),
    "tie_to_higher": ("if (best < 0 || scores[g] > scores[best])",
                      "if (best < 0 || scores[g] >= scores[best])"),
    "gqa_modulo": ("const int hk = h / ratio;", "const int hk = h % Hkv;"),
    "scale_dropped": ("s *= scale;", "(void)scale;"),
    "lse_without_max": ("lse[r] = mx + log(l);", "lse[r] = log(l);"),
    "not_causal_self": ("for (int64_t j = 0; j <= i; ++j) {\n                int in_window",
                        "for (int64_t j = 0; j < i; ++j) {\n                int in_window"),
    "lower_set_highest": ("for (int x = 0; x < g; ++x) {", "for (int x = g - 1; x >= 0; --x) {"),
    "lower_code_swapped": ("code += binom(low[i - 1], i);", "code += binom(low[r - i], i);"),
    "kept_two_at_top4": ("return K <= 16 ? 3 : 2;", "return 2;"),
    "code_sizes_dropped": ("code += binom(g, j);", "code += 0 * binom(g, j);"),
    "count_far_edge": ("int64_t far_end = i - w;", "int64_t far_end = i - w + 1;"),
    "value_index": ("acc[e] += p * widen(v, is_bf16, vb + e);",
                    "acc[e] += p * widen(v, is_bf16, kb_unused(vb) + e);"),
    "project_fma": ("float p = W[(int64_t)j * dm + e] * load_as_f32(x, is_bf16, t * dm + e);\n"
                    "                s = s + p;",
                    "s = fmaf(W[(int64_t)j * dm + e], load_as_f32(x, is_bf16, t * dm + e), s);"),
    "project_w_transposed": ("W[(int64_t)j * dm + e]", "W[(int64_t)e * 16 + j]"),
    "project_reverse_order": ("for (int e = 0; e < dm; ++e) {\n                float p = W",
                              "for (int e = dm - 1; e >= 0; --e) {\n                float p = W"),
    "bwd_dq_drop_d": ("const double ds = p * (dp - D);", "const double ds = p * dp;"),
    "bwd_dk_drop_d": ("const double ds = p * (dp - Ds[(int64_t)h * n + i]);",
                      "const double ds = p * dp;"),
    "bwd_dk_no_scale": ("dkj[e] += scale * ds * widen(q", "dkj[e] += ds * widen(q"),
    "bwd_dv_uses_ds": ("dvj[e] += p * widen(dout", "dvj[e] += ds * widen(dout"),
    "bwd_gqa_first_head_only": ("h < (int)(hk + 1) * ratio; ++h)", "h < (int)hk * ratio + 1; ++h)"),
    "bwd_window_le": ("if (!((i - j) < w || (bk[i] & bk[j]) != 0))",
                      "if (!((i - j) <= w || (bk[i] & bk[j]) != 0))"),
    "bwd_d_unnormalised": ("dd += widen(dout, is_bf16, dob + e) * (acc[e] / l);",
                           "dd += widen(dout, is_bf16, dob + e) * acc[e];"),
    "sinkhorn_skip_columns": ("Ah[t * K + g] *= ((double)n / K) / col[g];",
                              "Ah[t * K + g] *= 1.0 + 0.0 * col[g];"),
    "sinkhorn_rows_first": ("            /* columns to n / K */\n",
                            "            for (int64_t t = 0; t < n; ++t) { double rs = 0.0;"
                            " for (int g = 0; g < K; ++g) rs += Ah[t * K + g];"
                            " for (int g = 0; g < K; ++g) Ah[t * K + g] /= rs; }\n"
                            "            if (it == iters - 1) break;\n"),
    "gate_on_window_pairs": ("                if (i - j >= w) {\n                    const double *Aj",
                             "                if (1) {\n                    const double *Aj"),
    "gate_sign": ("gate = 1.0 / (1.0 + exp(-lambda * a));", "gate = 1.0 / (1.0 + exp(lambda * a));"),
    "affinity_first_group_only": ("                    for (int g = 0; g < K; ++g)\n"
                                  "                        a += Ai[g] * Aj[g];",
                                  "                    for (int g = 0; g < 1; ++g)\n"
                                  "                        a += Ai[g] * Aj[g];"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    assert SRC.count(old) >= 1, f"mutation site for {name} not found"
    src = SRC.replace(old, new)
    if name == "value_index":   # read v at the query row instead of the key row
        src = src.replace("static double widen(",
                          "#define kb_unused(x) (((int64_t)hk * n + i) * d)\nstatic double widen(")
    cfile = tmp_path / "mut.c"
    cfile.write_text(src)
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    "-std=c11", str(cfile), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, FOCUS_ORACLE_LIB=str(lib))
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          str(ROOT / "tests" / "test_oracle_pins.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"pins did not catch mutation {name}:\n{res.stdout[-2000:]}"
