"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin takes the loaded oracle library and raises AssertionError on a
mismatch.  The pytest file runs every pin on the real oracle, and runs the
whole battery on deliberately broken copies of oracle.c to show that each
plausible mistake is caught by at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle
from tests import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _close(a, b, rtol=1e-10, atol=1e-12, what=""):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    if a.shape != b.shape or not np.allclose(a, b, rtol=rtol, atol=atol):
        err = np.max(np.abs(a - b)) if a.shape == b.shape else "shape"
        raise AssertionError(f"{what}: mismatch (max abs err {err})")


def _bits(x) -> np.ndarray:
    x = np.asarray(x, np.float32)
    b = W.f32_to_bf16_bits(x).reshape(x.shape)
    assert np.array_equal(W.bf16_bits_to_f32(b).reshape(x.shape), x), "fixture value not exact in bf16"
    return b


# --------------------------------------------------------------------- golden closed forms
def pin_golden_closed_forms(lib):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    env = {"e": math.e, "__builtins__": {}}
    for c in cases:
        q = _bits(c["q"])[None]                # [1, Hq, D]
        k = _bits(c["k"])[None]                # [1, Hkv, S, D]
        v = _bits(c["v"])[None]
        lens = np.array([c["len"]], np.int32)
        out = oracle.decode(q, k, v, lens, c["scale"], lib=lib)[0]
        exp = np.array([[eval(s, env) for s in row] for row in c["expected"]], np.float64)
        _close(out, exp, what=c["name"])


# --------------------------------------------------------------------- library special case
def _sdpa_reference(case: W.Case) -> np.ndarray:
    """torch scaled_dot_product_attention (CPU, float64), heads repeated per kv head."""
    q = torch.from_numpy(W.bf16_bits_to_f32(case.q).reshape(case.q.shape).astype(np.float64))
    k = torch.from_numpy(W.bf16_bits_to_f32(case.k).reshape(case.k.shape).astype(np.float64))
    v = torch.from_numpy(W.bf16_bits_to_f32(case.v).reshape(case.v.shape).astype(np.float64))
    out = np.zeros((case.B, case.Hq, case.D))
    for b in range(case.B):
        n = int(case.seq_lens[b])
        if n == 0:
            continue
        kb = k[b, :, :n].repeat_interleave(case.G, dim=0)[None]   # [1, Hq, n, D]
        vb = v[b, :, :n].repeat_interleave(case.G, dim=0)[None]
        qb = q[b][None, :, None, :]                               # [1, Hq, 1, D]
        o = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, scale=case.scale)
        out[b] = o[0, :, 0, :].numpy()
    return out


def pin_torch_sdpa(lib):
    cases = [
        W.contig_case(1, 8, 2, 64, 96, seed=1),
        W.contig_case(2, 6, 1, 128, 77, seq_lens=[77, 40], seed=2),
        W.contig_case(3, 12, 3, 32, 33, seq_lens=[1, 33, 17], seed=3),
        W.contig_case(1, 24, 4, 256, 64, seed=4, scale=1.0 / 16),
        W.contig_case(2, 4, 4, 16, 20, seq_lens=[20, 0], seed=5),
    ]
    for c in cases:
        _close(oracle.decode(c.q, c.k, c.v, c.seq_lens, c.scale, lib=lib), _sdpa_reference(c),
               what=f"sdpa B={c.B} Hq={c.Hq} Hkv={c.Hkv} D={c.D}")


# --------------------------------------------------------------------- brute force
def pin_brute_force(lib):
    """Pure-Python softmax with correctly rounded sums (math.fsum) on tiny inputs."""
    c = W.contig_case(2, 4, 2, 8, 6, seq_lens=[6, 3], seed=7, scale=0.37)
    q = W.bf16_bits_to_f32(c.q).reshape(c.q.shape).astype(float)
    k = W.bf16_bits_to_f32(c.k).reshape(c.k.shape).astype(float)
    v = W.bf16_bits_to_f32(c.v).reshape(c.v.shape).astype(float)
    exp = np.zeros((c.B, c.Hq, c.D))
    for b in range(c.B):
        n = int(c.seq_lens[b])
        for h in range(c.Hq):
            kv = h // c.G
            s = [c.scale * math.fsum(q[b, h, d] * k[b, kv, t, d] for d in range(c.D))
                 for t in range(n)]
            z = [math.exp(x) for x in s]
            Z = math.fsum(z)
            for d in range(c.D):
                exp[b, h, d] = math.fsum(z[t] * v[b, kv, t, d] for t in range(n)) / Z
    _close(oracle.decode(c.q, c.k, c.v, c.seq_lens, c.scale, lib=lib), exp, what="brute force")


# --------------------------------------------------------------------- closed-form invariants
def pin_len_one_is_v0(lib):
    c = W.contig_case(2, 8, 2, 64, 5, seq_lens=[1, 1], seed=8)
    out = oracle.decode(c.q, c.k, c.v, c.seq_lens, c.scale, lib=lib)
    v0 = W.bf16_bits_to_f32(c.v[:, :, 0, :]).reshape(c.B, c.Hkv, c.D).astype(np.float64)
    exp = np.repeat(v0, c.G, axis=1)
    if not np.array_equal(out, exp):
        raise AssertionError("len=1 must return V[0] exactly")


def pin_uniform_weights_give_mean(lib):
    """Identical keys, q = 0 or scale = 0 all give the plain mean of V[0:len]."""
    base = W.contig_case(1, 4, 2, 32, 40, seq_lens=[37], seed=9)
    vf = W.bf16_bits_to_f32(base.v).reshape(base.v.shape).astype(np.float64)
    mean = np.repeat(vf[0, :, :37, :].mean(axis=1), base.G, axis=0)[None]
    same_k = base.k.copy()
    same_k[:, :, :, :] = base.k[:, :, :1, :]
    _close(oracle.decode(base.q, same_k, base.v, base.seq_lens, base.scale, lib=lib), mean,
           what="identical keys")
    _close(oracle.decode(np.zeros_like(base.q), base.k, base.v, base.seq_lens, base.scale, lib=lib),
           mean, what="q = 0")
    _close(oracle.decode(base.q, base.k, base.v, base.seq_lens, 0.0, lib=lib), mean,
           what="scale = 0")


def pin_dominant_key(lib):
    """One score above every other by >= 60 returns that row of V (within n e^-60)."""
    c = W.contig_case(1, 2, 1, 16, 50, seed=10, scale=1.0)
    q = np.zeros_like(c.q)
    q[0, :, 0] = _bits([4.0])[0]
    k = np.zeros_like(c.k)
    k[0, 0, :, 0] = _bits((np.arange(50) % 9 - 4).astype(np.float32) / 4)
    k[0, 0, 23, 0] = _bits([16.0])[0]            # score 64, others <= 4
    out = oracle.decode(q, k, c.v, c.seq_lens, c.scale, lib=lib)
    v23 = W.bf16_bits_to_f32(c.v[0, 0, 23]).astype(np.float64)
    _close(out[0, 0], v23, rtol=0, atol=50 * math.exp(-60) * 10, what="dominant key")
    _close(out[0, 1], v23, rtol=0, atol=50 * math.exp(-60) * 10, what="dominant key")


def pin_scale_moves_into_q(lib):
    """(2q, scale/2) equals (q, scale) exactly: the scale multiplies the dot product."""
    c = W.contig_case(1, 8, 2, 64, 64, seed=11)
    qf = W.bf16_bits_to_f32(c.q).reshape(c.q.shape)
    q2 = W.f32_to_bf16_bits(qf * np.float32(2)).reshape(c.q.shape)
    a = oracle.decode(c.q, c.k, c.v, c.seq_lens, c.scale, lib=lib)
    b = oracle.decode(q2, c.k, c.v, c.seq_lens, c.scale / 2, lib=lib)
    if not np.array_equal(a, b):
        raise AssertionError("(2q, scale/2) must equal (q, scale)")
    c3 = oracle.decode(c.q, c.k, c.v, c.seq_lens, c.scale * 2, lib=lib)
    if np.allclose(a, c3, rtol=1e-6, atol=1e-9):
        raise AssertionError("the scale must change the result")


def pin_v_is_linear(lib):
    """Doubling V (exact in bf16) doubles the output exactly."""
    c = W.contig_case(1, 4, 1, 32, 30, seed=12)
    v2 = W.f32_to_bf16_bits(W.bf16_bits_to_f32(c.v) * np.float32(2)).reshape(c.v.shape)
    a = oracle.decode(c.q, c.k, c.v, c.seq_lens, c.scale, lib=lib)
    b = oracle.decode(c.q, c.k, v2, c.seq_lens, c.scale, lib=lib)
    if not np.array_equal(2 * a, b):
        raise AssertionError("out(2V) must equal 2 out(V)")


def pin_token_permutation(lib):
    """Reordering the tokens (K and V rows together) does not change the output."""
    c = W.contig_case(2, 6, 3, 64, 48, seq_lens=[48, 31], seed=13)
    rng = np.random.default_rng(99)
    k2, v2 = c.k.copy(), c.v.copy()
    for b in range(c.B):
        n = int(c.seq_lens[b])
        p = rng.permutation(n)
        k2[b, :, :n] = c.k[b][:, p]
        v2[b, :, :n] = c.v[b][:, p]
    _close(oracle.decode(c.q, c.k, c.v, c.seq_lens, c.scale, lib=lib),
           oracle.decode(c.q, k2, v2, c.seq_lens, c.scale, lib=lib), what="token permutation")


def pin_head_mapping(lib):
    """Swapping the data of kv heads i and j swaps the output head groups."""
    c = W.contig_case(1, 12, 3, 32, 40, seed=14)
    G = c.G
    k2, v2 = c.k.copy(), c.v.copy()
    k2[:, [0, 2]] = c.k[:, [2, 0]]
    v2[:, [0, 2]] = c.v[:, [2, 0]]
    q2 = c.q.copy()
    q2[:, 0:G], q2[:, 2 * G:3 * G] = c.q[:, 2 * G:3 * G], c.q[:, 0:G]
    a = oracle.decode(c.q, c.k, c.v, c.seq_lens, c.scale, lib=lib)
    b = oracle.decode(q2, k2, v2, c.seq_lens, c.scale, lib=lib)
    exp = a.copy()
    exp[:, 0:G], exp[:, 2 * G:3 * G] = a[:, 2 * G:3 * G], a[:, 0:G]
    if not np.array_equal(b, exp):
        raise AssertionError("head groups must follow their kv head")


def pin_nan_tail_ignored(lib):
    """Rows at or beyond len (here NaN or inf) never reach the output."""
    lens = [5, 17, 0]
    a = W.contig_case(3, 4, 2, 64, 24, seq_lens=lens, seed=15)
    for tail in ("nan", "inf"):
        b = W.contig_case(3, 4, 2, 64, 24, seq_lens=lens, seed=15, tail=tail)
        oa = oracle.decode(a.q, a.k, a.v, a.seq_lens, a.scale, lib=lib)
        ob = oracle.decode(b.q, b.k, b.v, b.seq_lens, b.scale, lib=lib)
        if not np.array_equal(oa, ob):
            raise AssertionError(f"{tail} tail changed the output")
        if not np.all(ob[2] == 0):
            raise AssertionError("len = 0 must give a zero row")


def pin_split_invariance(lib):
    """Split partials folded by the log-sum-exp rescale equal the one-pass result."""
    c = W.contig_case(2, 8, 2, 64, 150, seq_lens=[150, 61], seed=16)
    full = oracle.decode(c.q, c.k, c.v, c.seq_lens, c.scale, lib=lib)
    for chunk in (1, 2, 3, 7, 64, 150, 1000):
        part = oracle.decode(c.q, c.k, c.v, c.seq_lens, c.scale, chunk=chunk, lib=lib)
        _close(part, full, rtol=1e-12, atol=1e-14, what=f"split chunk={chunk}")
    # scores of several hundred: every exponent must be taken relative to a running max
    big = W.contig_case(1, 4, 1, 64, 90, seed=20, scale=100.0)
    full = oracle.decode(big.q, big.k, big.v, big.seq_lens, big.scale, lib=lib)
    if not np.all(np.isfinite(full)):
        raise AssertionError("large scores must not overflow")
    for chunk in (4, 30):
        part = oracle.decode(big.q, big.k, big.v, big.seq_lens, big.scale, chunk=chunk, lib=lib)
        _close(part, full, rtol=1e-12, atol=1e-14, what=f"large-score split chunk={chunk}")
    p = W.paged_case(3, 8, 2, 32, 16, 40, seq_lens=[150, 1, 77], seed=17)
    full = oracle.paged_decode(p.q, p.k, p.v, p.seq_lens, p.page_table, p.scale, lib=lib)
    for chunk in (1, 5, 16, 33):
        part = oracle.paged_decode(p.q, p.k, p.v, p.seq_lens, p.page_table, p.scale, chunk=chunk,
                                   lib=lib)
        _close(part, full, rtol=1e-12, atol=1e-14, what=f"paged split chunk={chunk}")


def gather_pages(p: W.Case):
    """Copy a paged cache into a contiguous [B, Hkv, max_pages*ps, D] cache (data movement only)."""
    S = p.max_pages * p.page_size
    k = np.zeros((p.B, p.Hkv, S, p.D), np.uint16)
    v = np.zeros_like(k)
    for b in range(p.B):
        for i in range(p.max_pages):
            pg = int(p.page_table[b, i])
            if pg < 0:
                continue
            k[b, :, i * p.page_size:(i + 1) * p.page_size] = p.k[pg]
            v[b, :, i * p.page_size:(i + 1) * p.page_size] = p.v[pg]
    return k, v


def pin_paged_equals_gathered(lib):
    p = W.paged_case(4, 8, 2, 64, 16, 64, seq_lens=[1, 16, 17, 200], max_len=256, seed=18)
    k, v = gather_pages(p)
    a = oracle.paged_decode(p.q, p.k, p.v, p.seq_lens, p.page_table, p.scale, lib=lib)
    b = oracle.decode(p.q, k, v, p.seq_lens, p.scale, lib=lib)
    if not np.array_equal(a, b):
        raise AssertionError("paged must equal the gathered contiguous cache")


def pin_page_permutation(lib):
    """Moving pages to other pool slots (table updated to match) gives identical output."""
    p = W.paged_case(3, 8, 4, 32, 8, 60, seq_lens=[100, 7, 64], max_len=128, seed=19)
    rng = np.random.default_rng(5)
    perm = rng.permutation(p.num_pages)           # new slot of old page i
    k2 = np.empty_like(p.k)
    v2 = np.empty_like(p.v)
    k2[perm] = p.k
    v2[perm] = p.v
    t2 = np.where(p.page_table >= 0, perm[np.maximum(p.page_table, 0)], -1).astype(np.int32)
    a = oracle.paged_decode(p.q, p.k, p.v, p.seq_lens, p.page_table, p.scale, lib=lib)
    b = oracle.paged_decode(p.q, k2, v2, p.seq_lens, t2, p.scale, lib=lib)
    if not np.array_equal(a, b):
        raise AssertionError("page permutation changed the output")


# --------------------------------------------------------------------- the E4M3 cache
def _fp8_values(lib, v_scale=1.0) -> np.ndarray:
    """The oracle's value of every E4M3 byte (NaN bytes 0x7F / 0xFF read as NaN), through the
    len = 1 identity out = V[0]: the V row holds the 256 byte values."""
    D = 256
    q = _bits(np.zeros((1, 1, D), np.float32))
    k = np.zeros((1, 1, 1, D), np.uint8)
    row = np.arange(256, dtype=np.uint8)
    finite = (row != 0x7F) & (row != 0xFF)
    v = np.where(finite, row, 0).astype(np.uint8).reshape(1, 1, 1, D)
    out = oracle.decode_fp8(q, k, v, np.array([1], np.int32), 1.0, 1.0, v_scale, lib=lib)[0, 0]
    return np.where(finite, out, np.nan)


def pin_fp8_values(lib):
    """The E4M3 values the oracle dequantises to, against values of the OCP FP8 format:
    zero, the subnormal steps of 2^-9, every power of two 2^-6 .. 2^8, a few interior
    points, the maximum 448, strict growth over 0x00..0x7E and sign symmetry."""
    val = _fp8_values(lib)
    facts = {0x00: 0.0, 0x01: 2.0 ** -9, 0x02: 2.0 ** -8, 0x03: 3 * 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
             0x39: 1.125, 0x3C: 1.5, 0x3F: 1.875, 0x44: 3.0, 0x6F: 120.0, 0x7E: 448.0,
             0x80: 0.0, 0xB8: -1.0, 0xFE: -448.0}
    for e in range(1, 16):
        facts[e << 3] = 2.0 ** (e - 7)
    for b, x in facts.items():
        assert val[b] == x, f"E4M3 byte {b:#04x}: {val[b]} != {x}"
    pos = val[:0x7F]
    assert np.all(np.diff(pos) > 0), "E4M3 values must grow strictly over 0x00 .. 0x7E"
    assert np.array_equal(val[0x80:0xFF], -pos), "E4M3 sign bit must negate"
    assert np.isnan(val[0x7F]) and np.isnan(val[0xFF])
    half = _fp8_values(lib, v_scale=0.5)
    assert np.array_equal(half[:0x7F], pos * 0.5), "v_scale must multiply V"


def pin_fp8_values_match_torch(lib):
    """Every E4M3 byte the oracle dequantises against torch's float8_e4m3fn decode (a library
    implementation of the same OCP format: bias 7, subnormals at exponent 0, 0x7F / 0xFF NaN,
    no infinities)."""
    import torch
    val = _fp8_values(lib)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = ~np.isnan(ref)
    assert np.array_equal(np.isnan(val), ~finite), "NaN bytes differ from float8_e4m3fn"
    assert np.array_equal(val[finite], ref[finite]), "E4M3 values differ from float8_e4m3fn"


def _fp8_as_bf16(lib, case: W.Case) -> W.Case:
    """The same call with K and V dequantised (power-of-two scales: exact in bf16)."""
    table = _fp8_values(lib)
    kd = (table[case.k] * case.k_scale).astype(np.float32)
    vd = (table[case.v] * case.v_scale).astype(np.float32)
    return W.Case(case.name, case.B, case.Hq, case.Hkv, case.D, case.scale, case.q,
                  _bits(kd), _bits(vd), case.seq_lens, case.page_table, case.page_size)


def pin_fp8_matches_bf16(lib):
    """With power-of-two per-tensor scales every dequantised element is a bf16 value, so the
    E4M3 path must give exactly the bf16 path's output on the dequantised cache."""
    c = W.fp8_contig_case(2, 8, 2, 64, 40, seq_lens=[40, 17], seed=70, k_scale=0.5, v_scale=0.25)
    got = oracle.decode_fp8(c.q, c.k, c.v, c.seq_lens, c.scale, c.k_scale, c.v_scale, lib=lib)
    d = _fp8_as_bf16(lib, c)
    ref = oracle.decode(d.q, d.k, d.v, d.seq_lens, d.scale, lib=lib)
    assert np.array_equal(got, ref), "fp8 cache != bf16 cache holding the same values"
    p = W.fp8_paged_case(3, 8, 2, 64, 16, 40, seq_lens=[33, 1, 64], seed=71, k_scale=2.0,
                         v_scale=0.125)
    got = oracle.paged_decode_fp8(p.q, p.k, p.v, p.seq_lens, p.page_table, p.scale, p.k_scale,
                                  p.v_scale, lib=lib)
    d = _fp8_as_bf16(lib, p)
    ref = oracle.paged_decode(d.q, d.k, d.v, d.seq_lens, d.page_table, d.scale, lib=lib)
    assert np.array_equal(got, ref), "paged fp8 cache != bf16 cache holding the same values"


def pin_fp8_split_invariance(lib):
    c = W.fp8_contig_case(2, 8, 1, 64, 70, seq_lens=[70, 9], seed=72)
    ref = oracle.decode_fp8(c.q, c.k, c.v, c.seq_lens, c.scale, c.k_scale, c.v_scale, lib=lib)
    for chunk in (1, 3, 16, 70):
        got = oracle.decode_fp8(c.q, c.k, c.v, c.seq_lens, c.scale, c.k_scale, c.v_scale,
                                chunk=chunk, lib=lib)
        _close(got, ref, what=f"fp8 split chunk={chunk}")


# --------------------------------------------------------------------- multi-query rows
def pin_mq_rows_are_single_query_calls(lib):
    """Row (b, i) of a multi-query call is exactly the single-query call of query i over the
    first len - M + i + 1 keys (the causal limit), for contiguous and paged caches."""
    c = W.mq_case(3, 4, 8, 2, 64, 40, seq_lens=[40, 4, 21], seed=75)
    got = oracle.decode_mq(c.q, c.k, c.v, c.seq_lens, c.scale, lib=lib)
    for b in range(c.B):
        for i in range(c.M):
            n = int(c.seq_lens[b]) - c.M + i + 1
            ref = oracle.decode(c.q[b:b + 1, i], c.k[b:b + 1], c.v[b:b + 1],
                                np.array([n], np.int32), c.scale, lib=lib)
            assert np.array_equal(got[b, i], ref[0]), f"mq row b={b} i={i}"
    p = W.mq_paged_case(2, 3, 8, 2, 64, 16, 20, [37, 3], max_len=64, seed=76)
    got = oracle.paged_decode_mq(p.q, p.k, p.v, p.seq_lens, p.page_table, p.scale, lib=lib)
    for b in range(p.B):
        for i in range(p.M):
            n = int(p.seq_lens[b]) - p.M + i + 1
            ref = oracle.paged_decode(p.q[b:b + 1, i], p.k, p.v, np.array([n], np.int32),
                                      p.page_table[b:b + 1], p.scale, lib=lib)
            assert np.array_equal(got[b, i], ref[0]), f"paged mq row b={b} i={i}"


def pin_mq_torch_sdpa(lib):
    """Multi-query calls against torch scaled_dot_product_attention (CPU, float64) with a boolean
    mask holding the causal limit: query i of sequence b sees keys t <= len - M + i.  Rows with
    no visible key are zero in the oracle (SDPA leaves them undefined), checked apart."""
    for c in (W.mq_case(2, 4, 8, 2, 64, 40, seq_lens=[40, 9], seed=78),
              W.mq_case(1, 3, 6, 1, 128, 25, seq_lens=[25], seed=79, scale=0.2),
              W.mq_case(2, 5, 4, 4, 32, 12, seq_lens=[12, 2], seed=80)):
        got = oracle.decode_mq(c.q, c.k, c.v, c.seq_lens, c.scale, lib=lib)
        q = torch.from_numpy(W.bf16_bits_to_f32(c.q).reshape(c.q.shape).astype(np.float64))
        k = torch.from_numpy(W.bf16_bits_to_f32(c.k).reshape(c.k.shape).astype(np.float64))
        v = torch.from_numpy(W.bf16_bits_to_f32(c.v).reshape(c.v.shape).astype(np.float64))
        for b in range(c.B):
            n = int(c.seq_lens[b])
            limit = np.array([n - c.M + i + 1 for i in range(c.M)])   # keys visible to query i
            seen = limit > 0
            assert np.all(got[b][~seen] == 0), f"mq rows without keys must be zero (b={b})"
            if not seen.any():
                continue
            kb = k[b, :, :n].repeat_interleave(c.G, dim=0)[None]        # [1, Hq, n, D]
            vb = v[b, :, :n].repeat_interleave(c.G, dim=0)[None]
            qb = q[b].permute(1, 0, 2)[None]                             # [1, Hq, M, D]
            mask = torch.from_numpy(np.arange(n)[None, :] < limit[:, None])  # [M, n]
            o = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, attn_mask=mask, scale=c.scale)
            ref = o[0].permute(1, 0, 2).numpy()                          # [M, Hq, D]
            _close(got[b][seen], ref[seen], what=f"mq sdpa b={b} M={c.M} G={c.G} D={c.D}")


def pin_mq_future_keys_ignored(lib):
    """Changing the keys and values a query may not see (positions > len - M + i) leaves its
    row unchanged, and M = 1 is the single-query call."""
    c = W.mq_case(1, 5, 4, 1, 64, 30, seq_lens=[30], seed=77)
    base = oracle.decode_mq(c.q, c.k, c.v, c.seq_lens, c.scale, lib=lib)
    k, v = c.k.copy(), c.v.copy()
    k[:, :, 27:] = _bits(np.full(k[:, :, 27:].shape, 3.0, np.float32))
    v[:, :, 27:] = _bits(np.full(v[:, :, 27:].shape, -2.0, np.float32))
    moved = oracle.decode_mq(c.q, k, v, c.seq_lens, c.scale, lib=lib)
    assert np.array_equal(moved[0, :2], base[0, :2]), "rows 0-1 must not see keys >= 27"
    assert not np.array_equal(moved[0, 2:], base[0, 2:]), "rows 2-4 see key 27 and later"
    one = W.mq_case(2, 1, 8, 2, 64, 33, seq_lens=[33, 9], seed=78)
    assert np.array_equal(oracle.decode_mq(one.q, one.k, one.v, one.seq_lens, one.scale, lib=lib)[:, 0],
                          oracle.decode(one.q[:, 0], one.k, one.v, one.seq_lens, one.scale, lib=lib))


ALL_PINS = [
    pin_golden_closed_forms, pin_torch_sdpa, pin_brute_force, pin_len_one_is_v0,
    pin_uniform_weights_give_mean, pin_dominant_key, pin_scale_moves_into_q, pin_v_is_linear,
    pin_token_permutation, pin_head_mapping, pin_nan_tail_ignored, pin_split_invariance,
    pin_paged_equals_gathered, pin_page_permutation, pin_fp8_values, pin_fp8_values_match_torch,
    pin_fp8_matches_bf16,
    pin_fp8_split_invariance, pin_mq_rows_are_single_query_calls, pin_mq_torch_sdpa,
    pin_mq_future_keys_ignored,
]
