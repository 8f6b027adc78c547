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
    "dropped_weight": ("acc[d] += w * widen_bf16(vrow[d]);", "acc[d] += widen_bf16(vrow[d]);"),
    "dropped_normalisation": ("o[d] = acc[d] / l;", "o[d] = acc[d];"),
    "last_token_dropped": ("range_stats(L, qrow, b, kvh, 0, n, scale, s, &m, &l, acc);",
                           "range_stats(L, qrow, b, kvh, 0, n - 1 > 0 ? n - 1 : n, scale, s, &m, &l, acc);"),
    "page_offset_ignored": ("(size_t)(t / L->page_size)]", "(size_t)0]"),
    "page_row_transposed": ("(size_t)(t % L->page_size)) *", "(size_t)((t % L->page_size) ^ 1)) *"),
    "v_read_from_k": ("const uint16_t *vrow = L->v + row_offset", "const uint16_t *vrow = L->k + row_offset"),
    "split_weight_dropped": ("Lsum += w * l;", "Lsum += l;"),
    "split_max_ignored": ("double w = (m == -INFINITY) ? 0.0 : exp(m - M);",
                          "double w = (m == -INFINITY) ? 0.0 : exp(m);"),
    "q_row_of_other_head": ("q + ((size_t)b * Hq + h) * (size_t)D;",
                            "q + ((size_t)b * Hq + kvh) * (size_t)D;"),
    "k_dim_stride_transposed": ("dot += widen_bf16(q[d]) * widen_bf16(krow[d]);",
                                "dot += widen_bf16(q[d]) * widen_bf16(krow[(d * 7) % L->D]);"),
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
