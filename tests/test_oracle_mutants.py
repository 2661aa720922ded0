"""The pins are discriminating: each planted mistake in the oracle fails one.

Every case copies ``oracle/dsa_oracle.c``, applies one textual edit that a
plausible bug would make (a dropped term, a wrong sign, an off-by-one, a
wrong index, a reversed tie-break), builds the copy into a temporary shared
library, and runs every pin in ``test_oracle_pins`` against it.  At least one
pin must fail.  Mistakes are planted only in a throw-away copy, on the CPU.
"""
import inspect
import os
import shutil

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "dsa_oracle.c")

MUTANTS = {
    "relu_dropped": ("double relu = dot > 0.0 ? dot : 0.0;", "double relu = dot;"),
    "relu_after_weight": ("acc += wv * relu;", "acc += (wv * dot > 0.0 ? wv * dot : 0.0);"),
    "head_weight_index": ("(int64_t)r * HI + h);\n        acc", "(int64_t)r * HI);\n        acc"),
    "index_scale_dropped": ("= sh->idx_scale * accf;", "= accf;"),
    "causal_off_by_one": ("if (s > q_pos) {", "if (s >= q_pos) {"),
    "decode_alignment": ("const int32_t q_pos = L - sh->T + t;\n    for (int32_t s = 0; s < S; ++s) {\n      if",
                         "const int32_t q_pos = t;\n    for (int32_t s = 0; s < S; ++s) {\n      if"),
    # a ragged sequence's queries placed at the end of the whole cache
    "ragged_alignment": ("const int32_t q_pos = L - sh->T + t;", "const int32_t q_pos = S - sh->T + t;"),
    "fp8_scale_ignored": (" * ue8m0_value(sf[row * nblk + d / 128]);", ";"),
    "tie_break_reversed": ("return (a->index > b->index) - (a->index < b->index);",
                           "return (a->index < b->index) - (a->index > b->index);"),
    "nan_selectable": ("if (isnan(v) || (isinf(v) && v < 0)) continue;",
                       "if (isinf(v) && v < 0) continue;"),
    "pad_with_zero": ("for (int32_t j = take; j < Keff; ++j) out[j] = -1;",
                      "for (int32_t j = take; j < Keff; ++j) out[j] = 0;"),
    # cache fill and indexer inputs
    "rms_not_averaged": ("    ms /= ORC_FILL_LAT;\n", "\n"),
    "rope_turn_sign": ("kv[ORC_FILL_LAT + i] = a * c - b * s;", "kv[ORC_FILL_LAT + i] = a * c + b * s;"),
    "rope_pairs_in_place": ("kv[ORC_FILL_LAT + ORC_FILL_ROPE / 2 + i] = a * s + b * c;",
                            "kv[ORC_FILL_LAT + ORC_FILL_ROPE / 2 + i] = b;"),
    "layernorm_bias_dropped": ("* k_gamma[i] + k_beta[i];", "* k_gamma[i];"),
    "layernorm_sample_variance": ("var /= ORC_FILL_IDX;", "var /= (ORC_FILL_IDX - 1);"),
    "quant_scale_rounded_down": ("while (ldexp(448.0, e - 1) >= amax) --e;\n    while (ldexp(448.0, e) < amax) ++e;",
                                 "e = (int)floor(log2(amax / 448.0));"),
    "quant_scale_floor_dropped": ("if (e < -127) e = -127;", ""),
    "output_not_ascending": ("qsort(out, (size_t)take, sizeof(int32_t), by_value);", ""),
    "rotary_term_dropped": ("for (int32_t d = 0; d < D; ++d) /* latent part and rotary part together */",
                            "for (int32_t d = 0; d < sh->Dc; ++d)"),
    "softmax_scale_dropped": ("return (double)sh->sm_scale * dot;", "return dot;"),
    "value_columns_shifted": ("((int64_t)b * S + keys[j]) * D + d);", "((int64_t)b * S + keys[j]) * D + d + sh->Dr);"),
    "softmax_unnormalised": ("double p = keys[j] >= 0 ? exp(logit[j] - m) / l : 0.0;",
                             "double p = keys[j] >= 0 ? exp(logit[j] - m) : 0.0;"),
    "lse_missing_max": ("*lse = m + log(l);", "*lse = log(l);"),
    # absorption either side of the attention
    "absorb_head_stride": ("acc += qc[e] * kv_b[((int64_t)h * head_rows + e) * Dc + c];",
                           "acc += qc[e] * kv_b[((int64_t)h * Dn + e) * Dc + c];"),
    "absorb_output_key_half": ("kv_b + ((int64_t)h * head_rows + Dn + d) * Dc;",
                               "kv_b + ((int64_t)h * head_rows + d) * Dc;"),
    "absorb_query_rope_sign": ("qo[Dc + i] = a * cs - b * sn;", "qo[Dc + i] = a * cs + b * sn;"),
    "absorb_query_rope_interleaved": ("qo[Dc + i] = a * cs - b * sn;\n        qo[Dc + Dr / 2 + i] = a * sn + b * cs;",
                                      "qo[Dc + 2 * i] = a * cs - b * sn;\n        qo[Dc + 2 * i + 1] = a * sn + b * cs;"),
    "linear_transposed": ("bf16_value(W[(int64_t)j * Din + i]);", "bf16_value(W[(int64_t)i * Dout + j]);"),
    "invalid_index_as_key0": ("keys[j] = (s >= 0 && s < S) ? s : -1;", "keys[j] = (s >= 0 && s < S) ? s : 0;"),
}


def _pin_functions():
    return [f for name, f in inspect.getmembers(pins, inspect.isfunction)
            if name.startswith("test_") and f.__module__ == pins.__name__]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path, monkeypatch):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mut = tmp_path / "dsa_oracle.c"
    mut.write_text(src.replace(old, new))
    shutil.copy(os.path.join(os.path.dirname(SRC), "dsa_oracle.h"), tmp_path / "dsa_oracle.h")
    lib_path = str(tmp_path / "liboracle_mutant.so")
    oracle.build(src=str(mut), out=lib_path, extra=["-w", "-I", str(tmp_path)])
    monkeypatch.setattr(oracle, "LIB_PATH", lib_path)
    caught = []
    for fn in _pin_functions():
        params = inspect.signature(fn).parameters
        kwargs = {p: None for p in params}
        try:
            fn(**kwargs)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(fn.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"
