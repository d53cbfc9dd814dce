"""Each planted mistake in a copy of the oracle must make at least one pin fail.

The method follows the revert table of FreeToken PR #844 (Tests: each check is
run with only the logic it guards reverted and must fail); its conv-commit row
(the window restored one column early) is mutant ``history_not_shifted`` here.
Mistakes are planted in the oracle's C source on the CPU, never in GPU code.
"""
import os
import tempfile

import pytest

import oracle
from oracle_pins import PINS

MUTANTS = [
    ("conv_taps_reversed",
     "acc += r->cw[(size_t)c * W + w] * in;",
     "acc += r->cw[(size_t)c * W + (W - 1 - w)] * in;"),
    ("history_not_shifted",
     "r->hist[(size_t)w * C + c] = r->hist[(size_t)(w + 1) * C + c];",
     "r->hist[(size_t)w * C + c] = r->hist[(size_t)w * C + c];"),
    ("history_imported_reversed",
     "r->hist[(size_t)w * C + c] = ld(conv, ((size_t)slot * (W - 1) + w) * C + c, d->dtype);",
     "r->hist[(size_t)w * C + c] = ld(conv, ((size_t)slot * (W - 1) + (W - 2 - w)) * C + c, d->dtype);"),
    ("silu_sign",
     "acc = acc / (1.0 + exp(-acc));",
     "acc = acc / (1.0 + exp(acc));"),
    ("delta_sign",
     "const double u = b * (v[i] - a * r->Sk[i]);",
     "const double u = b * (v[i] + a * r->Sk[i]);"),
    ("delta_drops_alpha",
     "const double u = b * (v[i] - a * r->Sk[i]);",
     "const double u = b * (v[i] - r->Sk[i]);"),
    ("beta_on_v_only",
     "const double u = b * (v[i] - a * r->Sk[i]);",
     "const double u = b * v[i] - a * r->Sk[i];"),
    ("state_not_decayed",
     "S[(size_t)i * dk + j] = a * S[(size_t)i * dk + j] + u * kn[j];",
     "S[(size_t)i * dk + j] = S[(size_t)i * dk + j] + u * kn[j];"),
    ("output_uses_key",
     "s += S[(size_t)i * dk + j] * qn[j];",
     "s += S[(size_t)i * dk + j] * kn[j];"),
    ("output_scale_dropped",
     "o_t[(size_t)h * dv + i] = d->scale * s;",
     "o_t[(size_t)h * dv + i] = s;"),
    ("norm_without_sqrt",
     "double qs = 1.0 / sqrt(qq + d->l2_eps);",
     "double qs = 1.0 / (qq + d->l2_eps);"),
    ("key_norm_eps_dropped",
     "double ks = 1.0 / sqrt(kk + d->l2_eps);",
     "double ks = 1.0 / sqrt(kk);"),
    ("gqa_map_modulo",
     "const int kh = h / group;",
     "const int kh = h % HK;"),
    ("v_from_k_channels",
     "const double *v = r->y + (size_t)2 * HK * dk + (size_t)h * dv;",
     "const double *v = r->y + (size_t)HK * dk + (size_t)h * dv;"),
    ("state_read_untransposed",
     "(double)ssm[(((size_t)slot * HV + h) * dk + j) * dv + i];",
     "(double)ssm[(((size_t)slot * HV + h) * dv + i) * dk + j];"),
    ("verify_reads_batch_row_as_slot",
     "state_import(&r, d, ssm, conv, conv_w, slot);\n        for (int t = 0; t < rows; ++t) {",
     "state_import(&r, d, ssm, conv, conv_w, b);\n        for (int t = 0; t < rows; ++t) {"),
    ("commit_one_row_short",
     "for (int t = 0; t < n; ++t) {",
     "for (int t = 0; t < n - 1; ++t) {"),
    ("bf16_decode_shift",
     "uint32_t bits = ((uint32_t)h) << 16;",
     "uint32_t bits = ((uint32_t)h) << 15;"),
    ("gate_index_per_key_head",
     "const double a = ld(alpha, g_off + h, d->dtype);",
     "const double a = ld(alpha, g_off + kh, d->dtype);"),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name,before,after", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(source, name, before, after):
    assert source.count(before) == 1, "mutation site not found once: %s" % name
    with tempfile.TemporaryDirectory() as tmp:
        lib = oracle.compile_variant(source.replace(before, after), tmp)
        orc = oracle.Oracle(lib)
        failed = []
        for pin in PINS:
            try:
                pin(orc)
            except AssertionError:
                failed.append(pin.__name__)
        assert failed, "no pin caught mutant %s" % name
