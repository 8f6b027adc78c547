"""The CPU oracle against its pins (no GPU), and the pins against broken oracles."""
import os
import re
import shutil
import subprocess

import pytest

import oracle
from tests import oracle_pins

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)


# Plausible mistakes, each planted in a copy of oracle.c (on the CPU only).
MUTANTS = {
    "head_mapping_mod": ("const int kvh = h / G;", "const int kvh = h % Hkv;"),
    "dropped_scale": ("return scale * dot;", "return dot;"),
    "max_sign": ("double w = exp(s[t - t0] - m);", "double w = exp(m - s[t - t0]);"),
    "dropped_weight": ("acc[d] += w * v_elem(L, vbase + d);", "acc[d] += v_elem(L, vbase + d);"),
    "dropped_normalisation": ("o[d] = acc[d] / l;", "o[d] = acc[d];"),
    "last_token_dropped": ("range_stats(L, qrow, b, kvh, 0, n, scale, s, &m, &l, acc);",
                           "range_stats(L, qrow, b, kvh, 0, n - 1 > 0 ? n - 1 : n, scale, s, &m, &l, acc);"),
    "page_offset_ignored": ("(size_t)(t / L->page_size)]", "(size_t)0]"),
    "page_row_transposed": ("(size_t)(t % L->page_size)) *", "(size_t)((t % L->page_size) ^ 1)) *"),
    "v_read_from_k": ("acc[d] += w * v_elem(L, vbase + d);", "acc[d] += w * k_elem(L, vbase + d);"),
    "split_weight_dropped": ("Lsum += w * l;", "Lsum += l;"),
    "split_max_ignored": ("double w = (m == -INFINITY) ? 0.0 : exp(m - M);",
                          "double w = (m == -INFINITY) ? 0.0 : exp(m);"),
    "q_row_of_other_head": ("q + (((size_t)b * M + i) * Hq + h) * (size_t)D;",
                            "q + (((size_t)b * M + i) * Hq + kvh) * (size_t)D;"),
    # multi-query rows
    "mq_causal_off_by_one": ("const int n = seq_lens[b] - M + i + 1;", "const int n = seq_lens[b] - M + i;"),
    "mq_not_causal": ("const int n = seq_lens[b] - M + i + 1;", "const int n = seq_lens[b];"),
    "mq_query_order_reversed": ("q + (((size_t)b * M + i) * Hq + h) * (size_t)D;",
                                "q + (((size_t)b * M + (M - 1 - i)) * Hq + h) * (size_t)D;"),
    "k_dim_stride_transposed": ("dot += widen_bf16(q[d]) * k_elem(L, kbase + d);",
                                "dot += widen_bf16(q[d]) * k_elem(L, kbase + (d * 7) % L->D);"),
    # the E4M3 cache
    "fp8_exponent_bias": ("return sign * ldexp(1.0 + (double)m / 8.0, e - 7);",
                          "return sign * ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "fp8_subnormal_as_normal": ("if (e == 0) return sign * ldexp((double)m / 8.0, -6);",
                                "if (e == 0) return sign * ldexp(1.0 + (double)m / 8.0, -7);"),
    "fp8_sign_dropped": ("const double sign = (byte & 0x80) ? -1.0 : 1.0;", "const double sign = 1.0;"),
    "fp8_k_scale_dropped": ("if (L->fp8) return L->k_scale * decode_e4m3", "if (L->fp8) return decode_e4m3"),
    "fp8_v_scale_for_k": ("if (L->fp8) return L->k_scale * decode_e4m3", "if (L->fp8) return L->v_scale * decode_e4m3"),
    "fp8_mantissa_bits": ("const int e = (byte >> 3) & 0xF, m = byte & 7;", "const int e = (byte >> 3) & 0xF, m = byte & 3;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new)
    path = tmp_path / "oracle_mut.c"
    path.write_text(mutated)
    so = str(tmp_path / "liboracle_mut.so")
    oracle.build(src=str(path), out=so)
    lib = oracle.load(so)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError) as e:   # ValueError: the oracle rejected its inputs
            caught.append(pin.__name__)
    assert caught, f"no pin catches the mutant {name}"
