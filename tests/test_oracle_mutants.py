"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of oracle/oracle_zero.c -- a dropped
term, a wrong sign, a transposed operand or index, an off-by-one -- builds
it, and runs the pin tests against that build (ORACLE_LIB); they must fail.
The unmodified copy must pass, so a failure is the mistake's, not the
harness's.  Nothing here touches the GPU or the product library.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle_zero.c")

PINS_MATH = ["tests/test_oracle_adamw.py", "tests/test_oracle_reduce.py"]
PINS_LAYOUT = ["tests/test_oracle_layout.py"]
PINS_ACCT = ["tests/test_oracle_accounting.py"]
PINS_CONVERT = ["tests/test_oracle_convert.py"]
PINS_CONTROL = ["tests/test_oracle_control.py"]
PINS_RESHARD = ["tests/test_oracle_reshard.py"]
PINS_DIM0 = ["tests/test_oracle_dim0.py"]
PINS_Q8 = ["tests/test_oracle_q8.py"]

# (name, original text, planted text, pin files that must catch it)
MUTANTS = [
    ("m_sign", "float mt = b1 * *m + c1 * g;", "float mt = b1 * *m - c1 * g;", PINS_MATH),
    ("v_not_squared", "c2 * (g * g)", "c2 * g", PINS_MATH),
    ("no_bias_correction_m", "float mhat = mt / bc1;", "float mhat = mt;", PINS_MATH),
    ("no_bias_correction_v", "float vhat = vt / bc2;", "float vhat = vt;", PINS_MATH),
    ("eps_inside_sqrt", "float den = sqrtf(vhat) + eps;", "float den = sqrtf(vhat + eps);", PINS_MATH),
    # last-bit changes: a reciprocal in place of a division, a contracted multiply-add
    ("bias_correction_by_reciprocal", "float mhat = mt / bc1;", "float mhat = mt * (1.0f / bc1);",
     PINS_MATH),
    ("update_by_reciprocal", "float u = mhat / den;", "float u = mhat * (1.0f / den);", PINS_MATH),
    ("m_update_fused", "float mt = b1 * *m + c1 * g;", "float mt = fmaf(b1, *m, c1 * g);",
     PINS_MATH),
    ("no_weight_decay", "float wt = *w * d - lr * u;", "float wt = *w - lr * u;", PINS_MATH),
    ("update_sign", "float wt = *w * d - lr * u;", "float wt = *w * d + lr * u;", PINS_MATH),
    ("betas_swapped", "out10[1] = (float)beta1;", "out10[1] = (float)beta2;", PINS_MATH),
    ("bias_step_off_by_one", "pow(beta1, (double)step)", "pow(beta1, (double)(step + 1))", PINS_MATH),
    ("decay_without_lr", "out10[9] = (float)(1.0 - lr * wd);", "out10[9] = (float)(1.0 - wd);", PINS_MATH),
    ("row_index_transposed", "grad_at(grads, gdt, (int64_t)k * ld + j)",
     "grad_at(grads, gdt, (int64_t)j * ld + k)", PINS_MATH),
    ("last_row_dropped", "for (int32_t k = 0; k < n; ++k) {", "for (int32_t k = 0; k < n - 1; ++k) {",
     PINS_MATH),
    ("average_not_applied", "float g = a * c[0];\n        ss += (double)g * (double)g;\n"
     "        adamw_element(g, &w[j], &m[j], &v[j], c);\n        wout[j]",
     "float g = a;\n        ss += (double)g * (double)g;\n"
     "        adamw_element(g, &w[j], &m[j], &v[j], c);\n        wout[j]", PINS_MATH),
    ("accumulate_ignored", "float r = accumulate ? acc[j] + a : a;", "float r = a;", PINS_MATH),
    ("overflow_never_set", "if (nonfinite(r)) bad = 1;", "(void)r;", PINS_MATH),
    ("bf16_truncates", "if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1;", "(void)lo;",
     PINS_CONVERT),
    ("bf16_ties_away", "(lo == 0x8000u && (hi & 1u))", "(lo == 0x8000u)", PINS_CONVERT),
    ("f16_widen_bias", "((e + 112u) << 23)", "((e + 111u) << 23)", PINS_CONVERT),
    ("f16_subnormal_shift", "shift = -e - 1;", "shift = -e;", PINS_CONVERT),
    ("layout_floor", "int64_t units = ceil_div(n, unit);", "int64_t units = n / unit;", PINS_LAYOUT),
    ("segment_offset", "quads[4 * count + 1] = s - a;\n                quads[4 * count + 2] = s - lo;",
     "quads[4 * count + 1] = s - a;\n                quads[4 * count + 2] = s - lo + 1;", PINS_LAYOUT),
    ("padding_segment_dropped", "    if (hi > s) {\n        if (count < cap) {\n            quads[4 * count + 0] = -1;",
     "    if (0 && hi > s) {\n        if (count < cap) {\n            quads[4 * count + 0] = -1;", PINS_LAYOUT),
    ("stage2_grads_unsharded", "case 2: return w + g / n_dp + o / n_dp;", "case 2: return w + g + o / n_dp;",
     PINS_ACCT),
    ("comm_factor", "double f = (n_dp - 1.0) / n_dp * n;", "double f = n;", PINS_ACCT),
    ("clip_without_sqrt", "double norm = sqrt(sumsq) * (double)s;", "double norm = sumsq * (double)s;",
     PINS_CONTROL),
    ("clip_ignores_scale", "double norm = sqrt(sumsq) * (double)s;", "double norm = sqrt(sumsq);",
     PINS_CONTROL),
    ("clip_amplifies", "return c < 1.0 ? (float)c : 1.0f;", "return (float)c;", PINS_CONTROL),
    ("scale_backoff_as_growth", "*scale = (float)((double)*scale * backoff);",
     "*scale = (float)((double)*scale * growth);", PINS_CONTROL),
    ("scale_count_not_reset", "        *good_steps = 0;\n        return;", "        return;",
     PINS_CONTROL),
    ("dynamic_scale_multiplied", "c[0] = (float)(hp6[5] / (double)*loss_scale);",
     "c[0] = (float)(hp6[5] * (double)*loss_scale);", PINS_CONTROL),
    ("reshard_rank_offset", "int64_t flat = (int64_t)dst_rank * dst_shard + j;",
     "int64_t flat = (int64_t)dst_rank * src_shard + j;", PINS_RESHARD),
    ("reshard_padding_not_zeroed", "} else {\n            memset(d, 0, (size_t)elem_bytes);",
     "} else {\n            memcpy(d, (const unsigned char *)src[0], (size_t)elem_bytes);",
     PINS_RESHARD),
    ("locate_inclusive_end", "i - flat_off[k] < len[k]", "i - flat_off[k] <= len[k]", PINS_RESHARD),
    ("locate_ignores_n", "if (i < 0 || i >= n) return -1;", "if (i < 0) return -1;", PINS_RESHARD),
    ("scatter_range_from_zero", "n_dst, INT64_MAX, begin + j, &off)", "n_dst, INT64_MAX, j, &off)",
     PINS_RESHARD),
    ("dim0_chunk_floor", "int64_t c = ceil_div(rows[i], n_dp);\n        int64_t first",
     "int64_t c = rows[i] / n_dp;\n        int64_t first", PINS_DIM0),
    ("dim0_layout_chunk_floor", "int64_t c = ceil_div(rows[i], n_dp);\n        /* every size",
     "int64_t c = rows[i] / n_dp;\n        /* every size", PINS_DIM0),
    ("dim0_row_offset_not_scaled", "quads[4 * count + 1] = first * cols[i];",
     "quads[4 * count + 1] = first;", PINS_DIM0),
    ("dim0_padding_dropped", "if (have < c && cols[i] > 0) {", "if (0) {", PINS_DIM0),
    ("dim0_size_not_aligned", "out2[1] = ceil_div(p, align) * align;", "out2[1] = p;", PINS_DIM0),
    ("fp32_rows_read_as_16bit", "if (gdt == ORA_FP32) return ((const float *)grads)[i];",
     "(void)0;", PINS_DIM0),
    ("q8_scale_128", "float s = amax / 127.0f;", "float s = amax / 128.0f;", PINS_Q8),
    ("q8_ties_away", "float r = rintf(grad_at(x, xdt, j) / s);",
     "float r = roundf(grad_at(x, xdt, j) / s);", PINS_Q8),
    ("q8_codes_times_the_scale", "float r = rintf(grad_at(x, xdt, j) / s);",
     "float r = rintf(grad_at(x, xdt, j) * s);", PINS_Q8),
    ("q8_codes_scaled_by_128", "float r = rintf(grad_at(x, xdt, j) / s);",
     "float r = rintf(grad_at(x, xdt, j) * (128.0f / amax));", PINS_Q8),
    # the other plausible reading: codes with the block's reciprocal 127 / absmax
    ("q8_codes_by_the_reciprocal", "float r = rintf(grad_at(x, xdt, j) / s);",
     "float r = rintf(grad_at(x, xdt, j) * (127.0f / amax));", PINS_Q8),
    # the exact quotient rounded to a code, skipping its rounding to binary32
    ("q8_codes_from_the_exact_quotient", "float r = rintf(grad_at(x, xdt, j) / s);",
     "float r = (float)rint((double)grad_at(x, xdt, j) / (double)s);", PINS_Q8),
    ("q8_zero_scale_codes", "if (s == 0.0f || isnan(s) || isinf(s)) {", "if (isnan(s) || isinf(s)) {",
     PINS_Q8),
    ("q8_dequant_block_off_by_one", "return (float)q[j] * scales[j / ORA_Q8_BLOCK];",
     "return (float)q[j] * scales[(j + 1) / ORA_Q8_BLOCK];", PINS_Q8),
    ("q8_nan_not_sticky", "if (isnan(a) || a > m) m = a;", "if (a > m) m = a;", PINS_Q8),
    ("q8_step_quantizes_m", "ora_q8_quantize(w, ORA_FP32, len, wq, wscales);",
     "ora_q8_quantize(m, ORA_FP32, len, wq, wscales);", PINS_Q8),
    ("gather_holes_not_zeroed", "else\n            memset(d, 0, (size_t)elem_bytes);",
     "else\n            memset(d, 1, (size_t)elem_bytes);", PINS_RESHARD),
    ("reshard_half_elements", "(const unsigned char *)src[r] + o * elem_bytes;",
     "(const unsigned char *)src[r] + o * 2;", PINS_RESHARD),
    ("v_decay_uses_beta1", "float vt = b2 * *v + c2 * (g * g);", "float vt = b1 * *v + c2 * (g * g);",
     PINS_MATH),
    ("decay_after_update", "float wt = *w * d - lr * u;", "float wt = (*w - lr * u) * d;", PINS_MATH),
    ("cast_from_old_master",
     "        adamw_element(g, &w[j], &m[j], &v[j], c);\n        wout[j] = narrow(w[j], wdt);\n    }\n"
     "    if (overflow",
     "        wout[j] = narrow(w[j], wdt);\n        adamw_element(g, &w[j], &m[j], &v[j], c);\n    }\n"
     "    if (overflow", PINS_MATH),
    ("skip_ignored", "    if (skip && *skip) return;\n    float c[10];\n    ora_adamw_scalars(hp6, step, c);\n    for",
     "    float c[10];\n    ora_adamw_scalars(hp6, step, c);\n    for", PINS_MATH),
    ("sum_started_from_plus_zero",
     "        float x = grad_at(grads, gdt, (int64_t)k * ld + j);\n        a = (k == 0) ? x : a + x;",
     "        float x = grad_at(grads, gdt, (int64_t)k * ld + j);\n        a = a + x;", PINS_MATH),
    ("reduce_sumsq_of_the_partial", "        acc[j] = r;\n        ss += (double)r * (double)r;",
     "        acc[j] = r;\n        ss += (double)a * (double)a;", PINS_MATH),
    ("step_sumsq_before_the_average",
     "        ss += (double)g * (double)g;\n        adamw_element(g, &w[j], &m[j], &v[j], c);\n        wout[j]",
     "        ss += (double)a * (double)a;\n        adamw_element(g, &w[j], &m[j], &v[j], c);\n        wout[j]",
     PINS_MATH),
    ("step_overflow_never_set",
     "        if (nonfinite(a)) bad = 1;\n        float g = a * c[0];\n        ss += (double)g * (double)g;\n"
     "        adamw_element(g, &w[j], &m[j], &v[j], c);\n        wout",
     "        float g = a * c[0];\n        ss += (double)g * (double)g;\n"
     "        adamw_element(g, &w[j], &m[j], &v[j], c);\n        wout", PINS_MATH),
    ("scale_interval_off_by_one", "if (*good_steps >= interval) {", "if (*good_steps > interval) {",
     PINS_CONTROL),
    ("q8_scale_rows_at_the_code_stride",
     "float x = dequant(gq + (int64_t)k * ld, gs + (int64_t)k * sld, j);",
     "float x = dequant(gq + (int64_t)k * ld, gs + (int64_t)k * (ld / ORA_Q8_BLOCK), j);", PINS_Q8),
    ("q8_absmax_signed", "float a = fabsf(grad_at(x, xdt, j));", "float a = grad_at(x, xdt, j);", PINS_Q8),
    ("gather_begin_ignored", "int32_t k = ora_flat_locate(flat_off, len, n_src, n, begin + j, &off);",
     "int32_t k = ora_flat_locate(flat_off, len, n_src, n, j, &off);", PINS_RESHARD),
    ("reshard_divides_by_the_new_shard", "int64_t r = flat / src_shard, o = flat % src_shard;",
     "int64_t r = flat / dst_shard, o = flat % dst_shard;", PINS_RESHARD),
    ("layout_offsets_shifted", "        if (offsets) offsets[i] = n;\n        n += numels[i];",
     "        n += numels[i];\n        if (offsets) offsets[i] = n;", PINS_LAYOUT),
    ("dim0_chunk_not_clamped", "        if (have > c) have = c;\n", "", PINS_DIM0),
    ("clip_norm_not_unscaled",
     "    if (sumsq && max_norm > 0.0) clip = ora_clip_coef(*sumsq, c[0], max_norm);",
     "    if (sumsq && max_norm > 0.0) clip = ora_clip_coef(*sumsq, 1.0f, max_norm);", PINS_CONTROL),
]


def _build(src_text, out_dir, name):
    c = os.path.join(out_dir, f"{name}.c")
    so = os.path.join(out_dir, f"{name}.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                    "-I", os.path.join(ROOT, "oracle"), "-o", so, c, "-lm"], check=True)
    return so


def _run_pins(so, files):
    env = dict(os.environ, ORACLE_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + files, cwd=ROOT, env=env, capture_output=True, text=True)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def results():
    src = open(SRC).read()
    jobs = [("unmodified", src,
             PINS_MATH + PINS_LAYOUT + PINS_ACCT + PINS_CONTROL + PINS_RESHARD + PINS_DIM0 + PINS_Q8,
             None)]
    for name, old, new, files in MUTANTS:
        assert src.count(old) == 1, f"mutant {name}: its target text must occur once in the oracle"
        jobs.append((name, src.replace(old, new), files, old))
    out = {}
    with tempfile.TemporaryDirectory() as d:
        sos = {name: _build(text, d, name) for name, text, _, _ in jobs}
        with ThreadPoolExecutor(max_workers=4) as ex:
            futs = {name: ex.submit(_run_pins, sos[name], files) for name, _, files, _ in jobs}
            for name, f in futs.items():
                out[name] = f.result()
    return out


def test_unmodified_copy_passes_the_pins(results):
    rc, log = results["unmodified"]
    assert rc == 0, log


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(results, name):
    rc, log = results[name]
    # a failed pin (exit 1) or a crash of the broken build (killed by a
    # signal) -- not a usage error or an empty collection
    assert rc == 1 or rc < 0, f"the pins did not catch mutant {name} (exit {rc}): {log}"
