"""Plausible mistakes planted in a COPY of the oracle, on the CPU, must each
fail at least one pin: evidence that the pins would catch such an error in the
real oracle (a dropped term, a wrong index or sign, a wrong rounding)."""
import os

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ks_oracle.c")

# (name, original text, planted text, occurrence index to replace or None for all)
MUTANTS = [
    ("eps_dropped", "float d = mean + eps;", "float d = mean;"),
    ("eps_outside_sqrt", "return (float)(1.0 / sqrt((double)d));",
     "return (float)(1.0 / (sqrt((double)mean) + (double)eps));"),
    ("sqrt_dropped", "return (float)(1.0 / sqrt((double)d));", "return (float)(1.0 / (double)d);"),
    ("mean_off_by_one", "float mean = ss / (float)hidden;", "float mean = ss / (float)(hidden + 1);"),
    ("abs_not_square", "sum_sq += v * v;  /* each square is exact in double */",
     "sum_sq += fabs(v);"),
    ("weight_dropped", "float u = t * load_elem(dtype, w, j);\n            store_elem(dtype, out",
     "float u = t;\n            store_elem(dtype, out"),
    ("weight_reversed", "float u = t * load_elem(dtype, w, j);\n            store_elem(dtype, out",
     "float u = t * load_elem(dtype, w, hidden - 1 - j);\n            store_elem(dtype, out"),
    ("fused_sub", "s[j] = load_elem(dtype, x, base + j) + load_elem(dtype, residual, base + j);\n            double v",
     "s[j] = load_elem(dtype, x, base + j) - load_elem(dtype, residual, base + j);\n            double v"),
    ("fused_residual_is_x", "store_elem(dtype, residual, base + j, s[j]);",
     "store_elem(dtype, residual, base + j, load_elem(dtype, x, base + j));"),
    ("fused_normalises_rounded_sum", "float t = s[j] * scale;",
     "float t = load_elem(dtype, residual, base + j) * scale;"),
    ("fused_no_weight", "float u = t * load_elem(dtype, w, j);\n            store_elem(dtype, x,",
     "float u = t;\n            store_elem(dtype, x,"),
    ("round_truncates", "double r = nearbyint(n);", "double r = trunc(n);"),
    ("round_ties_away", "double r = nearbyint(n);", "double r = round(n);"),
    ("no_subnormals", "    if (lead < f->emin)\n        lead = f->emin;          /* subnormal range: fixed quantum */",
     "    if (lead < f->emin)\n        return copysign(0.0, a);"),
    ("bias_off_by_one", "int bias = 1 - f->emin;\n    int frac_bits = f->prec - 1;",
     "int bias = 2 - f->emin;\n    int frac_bits = f->prec - 1;"),
    ("widen_bias_off_by_one", "int bias = 1 - f->emin;\n    uint32_t exp_all_ones",
     "int bias = -f->emin;\n    uint32_t exp_all_ones"),
    ("scale_in_fp32_sqrt_of_mean_only", "float d = mean + eps;               /* fp32 add */",
     "float d = mean + eps * 0.5f;"),
    ("swiglu_sigmoid_sign", "return (float)(1.0 / (1.0 + exp(-(double)g)));",
     "return (float)(1.0 / (1.0 + exp((double)g)));"),
    ("swiglu_halves_swapped", "float g = load_elem(dtype, x, r * 2 * d + j);\n            float u = load_elem(dtype, x, r * 2 * d + d + j);",
     "float u = load_elem(dtype, x, r * 2 * d + j);\n            float g = load_elem(dtype, x, r * 2 * d + d + j);"),
    ("swiglu_no_gate_factor", "float t = g * sigmoid32(g);", "float t = sigmoid32(g);"),
    ("swiglu_up_off_by_one", "float u = load_elem(dtype, x, r * 2 * d + d + j);",
     "float u = load_elem(dtype, x, r * 2 * d + d + (j + 1) % d);"),
    ("residual_oop_subtracts", "s[j] = load_elem(dtype, x, base + j) + load_elem(dtype, residual, base + j);\n            sum_sq += (double)s[j] * (double)s[j];",
     "s[j] = load_elem(dtype, x, base + j) - load_elem(dtype, residual, base + j);\n            sum_sq += (double)s[j] * (double)s[j];"),
    ("residual_oop_rounds_sum", "sum_sq += (double)s[j] * (double)s[j];",
     "store_elem(dtype, out, base + j, s[j]);   /* rounds s to the dtype */\n"
     "            s[j] = load_elem(dtype, out, base + j);\n            sum_sq += (double)s[j] * (double)s[j];"),
    ("residual_oop_no_weight", "store_elem(dtype, out, base + j, scaled * load_elem(dtype, w, j));",
     "store_elem(dtype, out, base + j, scaled);"),
    ("backward_sign", "double grad = rho * dyv * (double)load_elem(dtype, w, j) - coef * xv;",
     "double grad = rho * dyv * (double)load_elem(dtype, w, j) + coef * xv;"),
    ("backward_rho_squared", "double coef = rho * rho * rho * dot / (double)hidden;",
     "double coef = rho * rho * dot / (double)hidden;"),
    ("backward_dot_without_weight",
     "double gv = (double)load_elem(dtype, dy, base + j) * (double)load_elem(dtype, w, j);",
     "double gv = (double)load_elem(dtype, dy, base + j);"),
    ("backward_dw_without_rho", "dw_sum[j] += dyv * xv * rho;", "dw_sum[j] += dyv * xv;"),
    ("backward_dw_times_weight", "dw_sum[j] += dyv * xv * rho;",
     "dw_sum[j] += dyv * xv * rho * (double)load_elem(dtype, w, j);"),
    ("backward_eps_dropped", "double rho = 1.0 / sqrt(sum_sq / (double)hidden + (double)eps);",
     "double rho = 1.0 / sqrt(sum_sq / (double)hidden);"),
    ("backward_grad_without_weight", "double grad = rho * dyv * (double)load_elem(dtype, w, j) - coef * xv;",
     "double grad = rho * dyv - coef * xv;"),
    ("softmax_no_max_shift", "float z = load_elem(dtype, x, base + j) - m;",
     "float z = load_elem(dtype, x, base + j);"),
    ("softmax_max_never_updated", "else if (v > m)\n                m = v;", "else if (v < m)\n                m = v;"),
    ("softmax_z_in_double", "float z = load_elem(dtype, x, base + j) - m;",
     "double z = (double)load_elem(dtype, x, base + j) - (double)m;"),
    ("softmax_exp_sign", "e[j] = exp((double)z);", "e[j] = exp(-(double)z);"),
    ("softmax_divides_by_h", "(float)(e[j] / sum)", "(float)(e[j] / (double)hidden)"),
    ("softmax_sum_skips_last", "sum += e[j];", "if (j + 1 < hidden)\n                sum += e[j];"),
    ("softmax_output_shifted", "store_elem(dtype, out, base + j, (float)(e[j] / sum));",
     "store_elem(dtype, out, base + (j + 1) % hidden, (float)(e[j] / sum));"),
    ("softmax_quotient_unrounded_to_fp32", "store_elem(dtype, out, base + j, (float)(e[j] / sum));",
     "store_elem(dtype, out, base + j, (float)(e[j] / sum * (1.0 + 0x1p-30)));"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique or missing"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.load(oracle.build(str(mutated), str(tmp_path / "libmutant.so")))
    failure = pins.first_failure(lib)
    assert failure is not None, f"mutant {name} passed every pin"
