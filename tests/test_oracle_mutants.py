"""The oracle's pins must catch plausible mistakes.  Each case plants one
mistake in a copy of oracle/oracle.cpp (on the CPU), builds it, and runs the
pin tests that should notice it against the mutant (ORACLE_LIB).  A mutant
that passes its pins means the pins are too weak."""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.cpp")

STEP = "tests/test_oracle_step.py"
FMT = "tests/test_oracle_formats.py"
LAY = "tests/test_oracle_layout.py"
CONS = "tests/test_oracle_consumer.py"

# (name, original text, planted mistake, tests expected to fail)
MUTANTS = [
    ("adam_c1_is_beta1", "const float c1 = (float)(1.0 - hp->beta1);",
     "const float c1 = (float)(hp->beta1);", STEP),
    ("adam_m_sign", "const float mn = b1 * m[i] + c1 * gg;",
     "const float mn = b1 * m[i] - c1 * gg;", STEP),
    ("adam_v_no_square", "const float vn = b2 * v[i] + c2 * (gg * gg);",
     "const float vn = b2 * v[i] + c2 * gg;", STEP),
    ("adam_betas_swapped", "const float vn = b2 * v[i] + c2 * (gg * gg);",
     "const float vn = b1 * v[i] + c1 * (gg * gg);", STEP),
    ("adam_bias_index_t_minus_1", "for (int64_t k = 0; k < t; ++k) { pw1",
     "for (int64_t k = 1; k < t; ++k) { pw1", STEP),
    ("adam_bias_index_t_plus_1", "for (int64_t k = 0; k < t; ++k) { pw1",
     "for (int64_t k = 0; k <= t; ++k) { pw1", STEP),
    ("adam_eps_inside_sqrt", "const float d = std::sqrt(vh) + eps;",
     "const float d = std::sqrt(vh + eps);", STEP),
    ("adam_no_weight_decay", "const float pn = p[i] * wdf - (lr * mh) / d;",
     "const float pn = p[i] - (lr * mh) / d;", STEP),
    ("adam_ascent", "const float pn = p[i] * wdf - (lr * mh) / d;",
     "const float pn = p[i] * wdf + (lr * mh) / d;", STEP),
    ("adam_coupled_decay", "const float gg = u * coef;",
     "const float gg = u * coef + (float)hp->weight_decay * p[i];", STEP),
    ("adam_clip_ignored", "const float gg = u * coef;", "const float gg = u;", STEP),
    ("adam_no_unscale", "const float u = load_elem(g, gdtype, i) * inv; /* unscaled gradient */",
     "const float u = load_elem(g, gdtype, i);", STEP),
    ("adam_writeback_old_p", "p[i] = pn;\n        if (lp_out) store_lp(lp_out, lp_dtype, i, pn);",
     "if (lp_out) store_lp(lp_out, lp_dtype, i, p[i]);\n        p[i] = pn;", STEP),
    ("reduce_reverse_order", "for (int32_t k = 0; k < n_ranks; ++k) acc = acc +",
     "for (int32_t k = n_ranks - 1; k >= 0; --k) acc = acc +", STEP),
    ("reduce_avg_by_reciprocal", "red[i] = (op == OR_AVG) ? acc / (float)n_ranks : acc;",
     "red[i] = (op == OR_AVG) ? acc * (1.0f / (float)n_ranks) : acc;", STEP),
    ("reduce_avg_missing", "red[i] = (op == OR_AVG) ? acc / (float)n_ranks : acc;",
     "red[i] = acc;", STEP),
    ("overflow_misses_nan", "if (!std::isfinite(u)) ovf = 1;", "if (std::isinf(u)) ovf = 1;",
     STEP),
    ("norm_fp32_square", "s = s + (double)u * (double)u;", "s = s + (double)(u * u);", STEP),
    ("clip_without_epsilon", "const double c = max_norm / (std::sqrt(sumsq_total) + 1e-6);",
     "const double c = max_norm / std::sqrt(sumsq_total);", STEP),
    ("scaler_grows_to_inf", "if (s->loss_scale < 0x1p127f) s->loss_scale",
     "if (1) s->loss_scale", STEP),
    ("scaler_grows_late", "if (s->good_steps == s->window) {",
     "if (s->good_steps == s->window + 1) {", STEP),
    ("scaler_static_halves", "if (s->dynamic) {\n            const float h",
     "if (1) {\n            const float h", STEP),
    ("scaler_counts_skipped", "s->good_steps = 0;\n        return;",
     "s->good_steps = 0;\n        s->step += 1;\n        return;", STEP),
    ("int8_scale_128", "const float scale = amax / 127.0f;",
     "const float scale = amax / 128.0f;", STEP),
    ("int8_half_away_from_zero", "float r = std::nearbyint(load_elem(x, dtype, j) / scale);",
     "float r = std::round(load_elem(x, dtype, j) / scale);", STEP),
    ("int8_truncates", "float r = std::nearbyint(load_elem(x, dtype, j) / scale);",
     "float r = std::trunc(load_elem(x, dtype, j) / scale);", STEP),
    ("round_half_up", "if (rem > half || (rem == half && (n & 1ull))) n += 1;",
     "if (rem >= half) n += 1;", FMT),
    ("round_truncate", "if (rem > half || (rem == half && (n & 1ull))) n += 1;", "", FMT),
    ("f16_emin_off_by_one", "round_to_format(x, 11, -14, 15, 5)",
     "round_to_format(x, 11, -15, 15, 5)", FMT),
    ("f16_subnormal_scale", "v = std::ldexp((double)m, -24);", "v = std::ldexp((double)m, -25);",
     FMT),
    ("bf16_widen_shift", "return bits_f32((uint32_t)h << 16);",
     "return bits_f32((uint32_t)h << 15);", FMT),
    ("layout_floor_shard", "(total % n_ranks != 0 ? 1 : 0)", "0", LAY),
    ("layout_align_ignored", "if (shard % align != 0) shard += align - shard % align;", "", LAY),
    ("layout_offset_in_shard", "seg_off_in_shard[count] = lo - lo_r;",
     "seg_off_in_shard[count] = lo;", LAY),
    ("acct_z2_grads_replicated",
     "out[2] = (int64_t)P * total + (int64_t)G * shard + (int64_t)K * shard;",
     "out[2] = (int64_t)P * total + (int64_t)G * total + (int64_t)K * shard;", LAY),
    ("acct_z1_optim_replicated",
     "out[1] = (int64_t)P * total + (int64_t)G * total + (int64_t)K * shard;",
     "out[1] = (int64_t)P * total + (int64_t)G * total + (int64_t)K * total;", LAY),
    ("dequant_global_block_index", "scales[(int64_t)s * nb + i / block]", "scales[j / block]",
     CONS),
    ("dequant_slot_not_offset", "const int64_t j = (int64_t)s * slot_numel + i;",
     "const int64_t j = i;", CONS),
    ("dequant_divides", "const float x = (float)q[j] * scales[", "const float x = (float)q[j] / scales[",
     CONS),
    ("dequant_code_as_unsigned", "const float x = (float)q[j] * scales[",
     "const float x = (float)(uint8_t)q[j] * scales[", CONS),
    ("dequant_bf16_truncates", "if (dtype == OR_F32) static_cast<float*>(out)[j] = x;\n"
     "            else store_lp(out, dtype, j, x);",
     "if (dtype == OR_F32) static_cast<float*>(out)[j] = x;\n"
     "            else if (dtype == OR_BF16) static_cast<uint16_t*>(out)[j] = "
     "(uint16_t)(f32_bits(x) >> 16);\n            else store_lp(out, dtype, j, x);", CONS),
    ("accumulate_overwrites", "acc[i] = acc[i] + red;", "acc[i] = red;", CONS),
    ("accumulate_rank_by_rank",
     "        float red;\n        oracle_reduce(bufs, n_ranks, dtype, offset + i, 1, op, &red);\n"
     "        acc[i] = acc[i] + red;",
     "        for (int32_t k = 0; k < n_ranks; ++k) acc[i] = acc[i] + load_elem(bufs[k], dtype, "
     "offset + i);", CONS),
    ("q8_scales_of_rank0", "const float x = (float)q[k][i] * scales[k][i / block];",
     "const float x = (float)q[k][i] * scales[0][i / block];", CONS),
    ("q8_block_fixed_256", "const float x = (float)q[k][i] * scales[k][i / block];",
     "const float x = (float)q[k][i] * scales[k][i / 256];", CONS),
    ("q8_divides", "const float x = (float)q[k][i] * scales[k][i / block];",
     "const float x = (float)q[k][i] / scales[k][i / block];", CONS),
    ("q8_reverse_order", "for (int32_t k = 0; k < n_ranks; ++k) {\n            const float x",
     "for (int32_t k = n_ranks - 1; k >= 0; --k) {\n            const float x", CONS),
    ("q8_avg_missing", "acc = acc + x;\n        }\n        red[i] = (op == OR_AVG) ? acc / (float)n_ranks : acc;",
     "acc = acc + x;\n        }\n        red[i] = acc;", CONS),
    ("accumulate_avg_ignored",
     "oracle_reduce(bufs, n_ranks, dtype, offset + i, 1, op, &red);",
     "oracle_reduce(bufs, n_ranks, dtype, offset + i, 1, OR_SUM, &red);", CONS),
]


def _run_mutant(case, tmpdir):
    name, old, new, tests = case
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: " + name
    mutated = src.replace(old, new, 1)
    d = os.path.join(tmpdir, name)
    os.makedirs(d)
    cpp = os.path.join(d, "oracle.cpp")
    open(cpp, "w").write(mutated)
    open(os.path.join(d, "oracle.h"), "w").write(
        open(os.path.join(ROOT, "oracle", "oracle.h")).read())
    lib = os.path.join(d, "liboracle.so")
    r = subprocess.run(["g++", "-std=c++17", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
                        "-fno-fast-math", "-mfpmath=sse", "-w", "-o", lib, cpp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        return name, "build failed: " + r.stderr[-500:]
    env = dict(os.environ, ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        tests], cwd=ROOT, env=env, capture_output=True, text=True)
    return name, r.returncode


def test_pins_catch_planted_mistakes():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 2)) as ex:
            results = list(ex.map(lambda c: _run_mutant(c, tmp), MUTANTS))
    survivors = [(n, rc) for n, rc in results if rc != 1]
    assert not survivors, "mutants not caught by the pins (or broken): %r" % survivors
