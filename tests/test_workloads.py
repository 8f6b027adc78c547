"""The seeded input generators (no GPU)."""
import numpy as np
import torch

from tests import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000, dtype=np.float32) * 100,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, 1e-40, np.inf,
                                  -np.inf], np.float32),
                        (np.arange(1 << 16, dtype=np.uint32) << 16 | 0x8000).view(np.float32)])
    x = x[np.isfinite(x) | np.isinf(x)]
    x = x[~np.isnan(x)]
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16)
                          .to(torch.float32).numpy())


def test_seeds_reproduce():
    a = W.contig_case(2, 4, 2, 32, 20, seed=3)
    b = W.contig_case(2, 4, 2, 32, 20, seed=3)
    c = W.contig_case(2, 4, 2, 32, 20, seed=4)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.q, b.q)
    assert not np.array_equal(a.k, c.k)


def test_page_assignment_distinct_and_covering():
    p = W.paged_case(32, 8, 2, 16, 32, 10000, max_len=8192, seed=0)
    assert p.max_pages == 256
    assert p.seq_lens.min() >= 1 and p.seq_lens.max() <= 8192
    used = []
    for b in range(p.B):
        n = (int(p.seq_lens[b]) + 31) // 32
        assert np.all(p.page_table[b, :n] >= 0) and np.all(p.page_table[b, n:] == -1)
        used.extend(p.page_table[b, :n].tolist())
    assert len(used) == len(set(used))
    assert all(0 <= u < 10000 for u in used)


def test_peaky_rows_scaled_by_8():
    base = W.contig_case(1, 2, 1, 16, 1000, seed=0)
    pk = W.peaky_case(1, 2, 1, 16, 1000, seed=0)
    a = W.bf16_bits_to_f32(base.k).reshape(base.k.shape)
    b = W.bf16_bits_to_f32(pk.k).reshape(pk.k.shape)
    changed = np.where(np.any(a != b, axis=-1))[2]
    assert len(changed) == 10
    assert np.array_equal(b[0, 0, changed], a[0, 0, changed] * 8)
    assert np.array_equal(base.v, pk.v) and np.array_equal(base.q, pk.q)


def test_named_workload_shapes():
    c = W.make("tiny_gqa4_d64_ctx512")
    assert (c.B, c.Hq, c.Hkv, c.D, c.S_max, c.scale) == (1, 8, 2, 64, 512, 0.125)
    assert c.algorithmic_bytes() == 512 * 2 * 64 * 4 + 8 * 64 * 2 + 8 * 64 * 4


def test_e4m3_encoder():
    """Nearest E4M3 value, ties to an even mantissa, saturation at 448, NaN -> 0x7F."""
    x = np.array([0.0, 1.0, 1.0625, 1.1875, 448.0, 1e6, -1.0, 2.0 ** -9, 2.0 ** -10,
                  3 * 2.0 ** -10, np.nan, -0.0, 240.0, 232.0], np.float32)
    got = W.f32_to_e4m3_bytes(x)
    want = [0x00, 0x38, 0x38, 0x3A, 0x7E, 0x7E, 0xB8, 0x01, 0x00, 0x02, 0x7F, 0x80, 0x77, 0x76]
    assert got.tolist() == want
    # every finite byte value is encoded to itself
    grid = W._E4M3
    assert np.array_equal(W.f32_to_e4m3_bytes(grid.astype(np.float32)), np.arange(127, dtype=np.uint8))
    assert np.array_equal(W.f32_to_e4m3_bytes(-grid[1:].astype(np.float32)),
                          (np.arange(1, 127) | 0x80).astype(np.uint8))


def test_fp8_cases():
    c = W.fp8_contig_case(2, 8, 2, 64, 50, seq_lens=[50, 7], seed=3, tail="nan")
    assert c.kv == "fp8" and c.k.dtype == np.uint8 and c.k.shape == (2, 2, 50, 64)
    assert np.all(c.k[1, :, 7:, :] == 0x7F) and not np.any(c.k[0] == 0x7F)
    assert c.algorithmic_bytes() == 57 * 2 * 64 * 2 + 2 * 8 * 64 * 6
    p = W.fp8_paged_case(4, 8, 2, 64, 16, 64, max_len=100, seed=4)
    assert p.paged and p.k.dtype == np.uint8 and p.page_table.shape == (4, 7)


def test_random_parity_draws_are_valid():
    """The random-shape parity generator: every draw respects the library's limits, and the cases
    it builds have the drawn shapes and lengths (the GPU test compares them with the oracle)."""
    from tests import test_gpu_random as R
    for i in range(R.N_CASES):
        c = R.draw(i)
        assert c == R.draw(i)
        assert c["M"] * c["G"] <= 16 and c["page_size"] % 16 == 0
        assert len(c["lens"]) == c["B"] and all(0 <= n <= c["S_max"] for n in c["lens"])
        if i % 5:
            continue  # building every case takes half a minute; every fifth covers each kind
        case = R.build(c)
        assert case.B == c["B"] and case.Hq == c["G"] * c["Hkv"] and case.D == c["D"]
        assert case.M == c["M"] and list(case.seq_lens) == c["lens"]
        assert case.paged == ("paged" in c["kind"]) and case.kv == ("fp8" if c["kind"].startswith("fp8") else "bf16")
