"""The CPU oracle against its pins, and planted mistakes against the pins.

The pins live in ``tests/oracle_pins.py``.  The mutation test copies
``oracle/oracle.c``, plants one plausible mistake (a dropped term, a wrong
index, a transposed operand, an off-by-one bound, a wrong sign), compiles it,
runs every pin in a child process and requires at least one pin to fail.
"""
import os
import subprocess
import sys

import pytest

import oracle
from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


# (name, text in oracle.c, replacement); every mutant must stay in bounds.
MUTANTS = [
    ("softmax_no_max_shift", "double m = -INFINITY;", "double m = 0.0;"),
    ("softmax_z_unshifted", "z += exp(scores[e * heads + h] - m);", "z += exp(scores[e * heads + h]);"),
    ("softmax_not_normalised", "exp(scores[e * heads + h] - m) / z;", "exp(scores[e * heads + h] - m);"),
    ("softmax_end_off_by_one", "for (int64_t e = start; e < end; ++e)\n                z +=",
     "for (int64_t e = start; e + 1 < end; ++e)\n                z +="),
    ("aggregate_head_dropped_in_gather",
     "acc += weights[e * heads + h] *\n                           load_feat(feat, dtype, ((int64_t)col_idx[e] * heads + h)",
     "acc += weights[e * heads + h] *\n                           load_feat(feat, dtype, ((int64_t)col_idx[e] * heads)"),
    ("aggregate_weight_head0", "acc += weights[e * heads + h] *", "acc += weights[e * heads] *"),
    ("aggregate_end_off_by_one", "for (int64_t e = start; e < end; ++e)\n                    acc +=",
     "for (int64_t e = start; e + 1 < end; ++e)\n                    acc +="),
    ("aggregate_negative_zero_start", "double acc = 0.0;\n                for (int64_t e",
     "double acc = -0.0;\n                for (int64_t e"),
    ("sddmm_operands_swapped", "int64_t a = ((int64_t)dst_idx[e] * heads + h) * head_dim;",
     "int64_t a = ((int64_t)src_idx[e] * heads + h) * head_dim;"),
    ("sddmm_scale_dropped", "out[e * heads + h] = scale * acc;", "out[e * heads + h] = acc;"),
    ("sddmm_dim_off_by_one", "for (int d = 0; d < head_dim; ++d)\n                acc +=",
     "for (int d = 1; d < head_dim; ++d)\n                acc +="),
    ("bf16_decode_shift", "<< 16;", "<< 15;"),
    ("layer_query_row_wrong", "dst[e] = (int32_t)i;", "dst[e] = 0;"),
    ("layer_k_v_swapped", "scores, v, dtype, out);", "scores, k, dtype, out);"),
    # backward
    ("softmax_bwd_dot_dropped", "out[e * heads + h] = alpha[e * heads + h] * (grad[e * heads + h] - dot);",
     "out[e * heads + h] = alpha[e * heads + h] * grad[e * heads + h];"),
    ("softmax_bwd_sign", "out[e * heads + h] = alpha[e * heads + h] * (grad[e * heads + h] - dot);",
     "out[e * heads + h] = alpha[e * heads + h] * (grad[e * heads + h] + dot);"),
    ("agg_bwd_dweights_head0", "acc += grad[(i * heads + h) * head_dim + d] *\n                           load_feat(feat",
     "acc += grad[(i * heads) * head_dim + d] *\n                           load_feat(feat"),
    ("agg_bwd_dfeat_wrong_column", "int64_t j = col_idx[e];\n                for (int d = 0; d < head_dim; ++d)\n                    dfeat",
     "int64_t j = col_idx[row_ptr[i]];\n                for (int d = 0; d < head_dim; ++d)\n                    dfeat"),
    ("layer_bwd_dq_scale_dropped", "dq[(i * heads + h) * head_dim + d] = scale * gsum;",
     "dq[(i * heads + h) * head_dim + d] = gsum;"),
    ("layer_bwd_dk_reads_k", "scale * gs[e * heads + h] * load_feat(q, dtype, (i * heads + h) * head_dim + d);",
     "scale * gs[e * heads + h] * load_feat(k, dtype, (j * heads + h) * head_dim + d);"),
    ("layer_bwd_dv_weights_are_scores", "n_src, a, v, dtype, grad, ga, dv);", "n_src, s, v, dtype, grad, ga, dv);"),
    ("sddmm_bwd_scale_dropped", "double w = scale * grad[e * heads + h];", "double w = grad[e * heads + h];"),
    ("sddmm_bwd_grad_head0", "double w = scale * grad[e * heads + h];", "double w = scale * grad[e * heads];"),
    ("sddmm_bwd_dsrc_reads_src", "const void* in = to_dst ? src_feat : dst_feat;",
     "const void* in = to_dst ? src_feat : src_feat;"),
    ("sddmm_bwd_input_head_dropped", "load_feat(in, dtype, (in_row * heads + h) * head_dim + d)",
     "load_feat(in, dtype, (in_row * heads) * head_dim + d)"),
    ("softagg_bwd_weights_are_scores", "n_src, alpha, feat, dtype, grad, ga, dfeat);",
     "n_src, scores, feat, dtype, grad, ga, dfeat);"),
    # dense relation-biased attention block
    ("relblock_unbiased_variance", "var /= D;", "var /= (D - 1);"),
    ("relblock_eps_dropped", "/ sqrt(var + eps) * gamma[d]", "/ sqrt(var) * gamma[d]"),
    ("relblock_weight_transposed", "sq += xn[i * D + c] * wq[r * D + c];", "sq += xn[i * D + c] * wq[c * D + r];"),
    ("relblock_silu_dropped", "hid[p] = t / (1.0 + exp(-t));", "hid[p] = t;"),
    ("relblock_scale_dropped", "lg[j] = dot * scale + rb;", "lg[j] = dot + rb;"),
    ("relblock_mask_inverted", "if (mask[(b * N + i) * N + j] < 0.5) continue;",
     "if (mask[(b * N + i) * N + j] > 0.5) continue;"),
    ("relblock_residual_dropped", "out[(b * N + i) * D + r] = x[i * D + r] + s;", "out[(b * N + i) * D + r] = s;"),
    ("relblock_bias_head0", "rb += w2[h * P + p] * hid[p];", "rb += w2[p] * hid[p];"),
    # node projections
    ("linear_weight_transposed", "load_feat(w, w_dtype, (int64_t)n * K + k);", "load_feat(w, w_dtype, (int64_t)k * N + n);"),
    ("linear_bias_dropped", "double s = bias ? bias[n] : 0.0;", "double s = 0.0;"),
    ("linear_k_off_by_one", "for (int k = 0; k < K; ++k)\n                s += load_feat(x",
     "for (int k = 1; k < K; ++k)\n                s += load_feat(x"),
    ("linear_x_row_wrong", "s += load_feat(x, x_dtype, m * K + k)", "s += load_feat(x, x_dtype, k)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(tmp_path, name, old, new):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    lib = oracle.build(str(mut), str(tmp_path / "liboracle_mut.so"))
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "oracle_pins.py"), lib],
                       capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode > 0, f"planted mistake {name} passed every pin:\n{r.stdout}{r.stderr}"
    assert "Traceback" not in r.stderr, r.stderr
