"""CPU: each plausible mistake planted in a copy of the oracle's source must
make at least one pin fail.  This checks the pins, not the oracle."""
import os

import pytest

import oracle
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.lib_path()), "pkm_oracle.c")

MUTATIONS = {
    "transposed_wq": ("q += (double)wrow[d] * (double)x_b[d];",
                      "q += (double)M->wq[((int64_t)h * D + d) * D + f] * (double)x_b[d];"),
    "bn_no_sqrt": ("/ sqrt((double)M->var[pf] + M->eps)", "/ ((double)M->var[pf] + M->eps)"),
    "bn_no_eps": ("sqrt((double)M->var[pf] + M->eps)", "sqrt((double)M->var[pf])"),
    "bn_beta_sign": ("(double)M->beta[pf];", "-(double)M->beta[pf];"),
    "bn_mean_dropped": ("(q - (double)M->mean[pf])", "(q)"),
    "swapped_halves": ("const double *qp = qhat + p * half;", "const double *qp = qhat + (1 - p) * half;"),
    "flat_index_swapped": ("grid[c].i = (int64_t)idx0[i] * n + idx1[j];", "grid[c].i = (int64_t)idx1[j] * n + idx0[i];"),
    "second_half_dropped": ("grid[c].v = top0[i] + top1[j];", "grid[c].v = top0[i];"),
    "ties_to_higher_index": ("if (a->i < b->i) return -1;\n    if (a->i > b->i) return 1;",
                             "if (a->i < b->i) return 1;\n    if (a->i > b->i) return -1;"),
    "ascending_scores": ("if (a->v > b->v) return -1;\n    if (a->v < b->v) return 1;",
                         "if (a->v > b->v) return 1;\n    if (a->v < b->v) return -1;"),
    "softmax_unnormalised": ("w[j] /= sum;", "w[j] /= 1.0;"),
    "softmax_no_max_shift": ("w[j] = exp(top[j] - mx);", "w[j] = exp(top[j]);"),
    "gather_unweighted": ("out_b[d] += w[j] * value_at(M, rows[j], d);", "out_b[d] += value_at(M, rows[j], d);"),
    "e4m3_bias": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "e4m3_no_scale": ("* (double)M->scale[row];", ";"),
    "bf16_subnormal": ("v = ldexp((double)m / 128.0, -126);", "v = ldexp((double)m / 128.0, -127);"),
    "int4_unsigned": ("return (double)(v >= 8 ? v - 16 : v);", "return (double)v;"),
    "int4_nibble_order": ("(uint8_t)(d & 1 ? byte >> 4 : byte)", "(uint8_t)(d & 1 ? byte : byte >> 4)"),
    "candidate_count": ("    return c;\n}", "    return c - 1;\n}"),
    "half_topk_from_wrong_row": ("pkmo_topk_sorted(n, s + n, kk, t1, i1);", "pkmo_topk_sorted(n, s, kk, t1, i1);"),
    # stand-alone steps
    "select_half1_from_half0": ("        pkmo_topk_sorted(n, s + n, k, t1, i1);\n        pkmo_candidates_topk(n, k, t0, i0, t1, i1, k, tp, fl);",
                                "        pkmo_topk_sorted(n, s, k, t1, i1);\n        pkmo_candidates_topk(n, k, t0, i0, t1, i1, k, tp, fl);"),
    "select_softmax_of_half0": ("if (w) pkmo_softmax(k, tp, w + p * k);", "if (w) pkmo_softmax(k, t0, w + p * k);"),
    "gather_out_not_cleared": ("            out[b * M->D + d] = 0.0;\n        pkmo_gather_add", "        pkmo_gather_add"),
    "gather_rows_of_first_bag": ("pkmo_gather_add(M, R, rows + b * R, w + b * R, out + b * M->D);",
                                 "pkmo_gather_add(M, R, rows, w + b * R, out + b * M->D);"),
    "scores_second_half_from_first_set": ("const float *c = M->subkeys + (((int64_t)h * 2 + p) * n + j) * half;",
                                          "const float *c = M->subkeys + (((int64_t)h * 2 + 0) * n + j) * half;"),
    "running_var_biased": ("momentum * (var[i] * unbias);", "momentum * var[i];"),
    "running_momentum_reversed": ("rmean[i] = (1.0 - momentum) * rmean[i] + momentum * mean[i];",
                                  "rmean[i] = momentum * rmean[i] + (1.0 - momentum) * mean[i];"),
    # backward direction
    "bwd_softmax_no_centering": ("dtj[j] = wj[j] * (g[j] - wg);", "dtj[j] = wj[j] * g[j];"),
    "bwd_dqhat_halves_swapped": ("dqh[half + d] += dtj[j] * (double)c1[d];", "dqh[half + d] += dtj[j] * (double)c0[d];"),
    "bwd_dq_without_gamma": ("dq[f] = dqh[f] * (double)M->gamma[pf] * inv;", "dq[f] = dqh[f] * inv;"),
    "bwd_dx_transposed": ("J->dx[b * D + d] += dq[f] * (double)wrow[d];",
                          "J->dx[b * D + d] += dq[f] * (double)M->wq[((int64_t)h * D + d) * D + f];"),
    "bwd_dgamma_from_qhat": ("J->dgamma[pf] += dqh * J->xhat[at];", "J->dgamma[pf] += dqh * J->qhat[at];"),
    "bwd_dwq_skips_bn_scale": ("const double dq = dqh * scale;", "const double dq = dqh;"),
    "bwd_dsub_wrong_half": ("const double *qp = J->qhat + bh * D + p * half;",
                            "const double *qp = J->qhat + bh * D + (1 - p) * half;"),
    "bwd_dval_unweighted": ("J->dval[r * D + d] += J->w[bh * k + j] * (double)gb[d];",
                            "J->dval[r * D + d] += (double)gb[d];"),
    "bwd_g_from_first_row": ("acc += (double)gb[d] * value_at(M, rj[j], d);", "acc += (double)gb[d] * value_at(M, rj[0], d);"),
    # batch statistics
    "bs_unbiased_var": ("var[(int64_t)h * D + f] = ss / (double)B;", "var[(int64_t)h * D + f] = ss / (double)(B - 1);"),
    "bs_xhat_no_eps": ("/ sqrt(S->var[at] + M->eps);", "/ sqrt(S->var[at]);"),
    "bs_dq_without_mean_term": ("(dqh[at] - m1[hf] - xhat[at] * m2[hf])", "(dqh[at] - xhat[at] * m2[hf])"),
    "bs_dq_without_xhat_term": ("(dqh[at] - m1[hf] - xhat[at] * m2[hf])", "(dqh[at] - m1[hf])"),
}

PINS = [
    pins.pin_select,
    pins.pin_gather,
    pins.pin_running_update,
    pins.pin_hand_example,
    pins.pin_codecs,
    pins.pin_integer_ties,
    pins.pin_k_equals_1,
    pins.pin_softmax_large_scores,
    pins.pin_op_counts,
    lambda lib: pins.pin_against_flat_search(pins.synthetic.WORKLOADS["tiny"], lib=lib),
    lambda lib: pins.pin_against_flat_search(pins.synthetic.Workload("gb", 24, 64, 3, 20, 5, "f32", "random"),
                                             gamma_beta=True, lib=lib),
    lambda lib: pins.pin_against_flat_search(pins.synthetic.Workload("q", 24, 128, 2, 24, 8, "e4m3", "random"),
                                             seed=2, lib=lib),
    lambda lib: pins.pin_against_flat_search(pins.synthetic.Workload("q4", 24, 128, 2, 24, 8, "int4", "random"),
                                             seed=2, lib=lib),
    pins.pin_backward_identities,
    lambda lib: pins.pin_backward_autograd(pins.synthetic.Workload("gb", 24, 64, 3, 20, 5, "f32", "random"),
                                           gamma_beta=True, lib=lib),
    pins.pin_backward_finite_differences,
    lambda lib: pins.pin_batch_stats_autograd(pins.synthetic.Workload("bs", 24, 64, 3, 20, 5, "f32", "random"),
                                              lib=lib),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = oracle.load_library(oracle.compile_source(str(src), str(tmp_path / "libmutant.so")))
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, RuntimeError):
            return
    pytest.fail(f"no pin caught the planted mistake {name}")
