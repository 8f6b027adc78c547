"""The E4M3 (FP8) KV cache: HIP path against the CPU oracle through the C ABI (needs an MI355X).

Tolerance (elementwise): |gpu - oracle| <= 2e-3 + 2e-3 |oracle|, the fp32 output against the
fp64 oracle evaluated on the same E4M3 bytes and scales (the quantization itself is part of the
inputs, not of the error).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import decode_attention_04_amd as gd
from tests import workloads as W
from tests.gpu_util import DeviceCase, compare, oracle_out, require_gpu

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a).view(np.uint32)


# ------------------------------------------------------------------ the workload shapes in E4M3
FP8_WORKLOADS = {
    "fp8_gqa6_d256_ctx4096": lambda: W.fp8_contig_case(1, 24, 4, 256, 4096, scale=1 / 16, seed=0,
                                                       name="fp8_gqa6_d256_ctx4096"),
    "fp8_long_gqa8_d128_ctx128k": lambda: W.fp8_contig_case(1, 8, 1, 128, 131072, seed=0,
                                                            name="fp8_long_gqa8_d128_ctx128k"),
    "fp8_paged_gqa4_d128_ragged8k": lambda: W.fp8_paged_case(32, 32, 8, 128, 32, 10000,
                                                             max_len=8192, seed=0,
                                                             name="fp8_paged_gqa4_d128_ragged8k"),
    "fp8_batched_gqa8_d128_ctx4k": lambda: W.fp8_contig_case(16, 32, 4, 128, 4096, seed=0,
                                                             name="fp8_batched_gqa8_d128_ctx4k"),
}


@pytest.mark.parametrize("name", list(FP8_WORKLOADS))
def test_fp8_workloads(name):
    say(f"[fp8] workload {name}: generating")
    case = FP8_WORKLOADS[name]()
    dc = DeviceCase(case)
    outs = [dc.run_host() for _ in range(3)]
    say(f"[fp8] workload {name}: oracle")
    stats = compare(outs[0], oracle_out(case), name)
    say(f"[fp8] workload {name}: {stats}")
    for o in outs[1:]:
        assert np.array_equal(_bits(o), _bits(outs[0])), "not bit-exact across runs"


# ------------------------------------------------------------------ shapes, tails, splits
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 2), (12, 2), (16, 1)])
def test_fp8_matrix_ragged_with_nan_tail(D, Hq, Hkv):
    lens = [1, 15, 17, 53, 517]
    say(f"[fp8] matrix D={D} Hq={Hq} Hkv={Hkv}")
    case = W.fp8_contig_case(len(lens), Hq, Hkv, D, 600, seq_lens=lens, seed=80 + D + Hq,
                             tail="nan")
    dc = DeviceCase(case)
    ref = oracle_out(case)
    for splits in (0, 1, 3, 40):
        compare(dc.run_host(splits), ref, f"fp8 D={D} Hq={Hq} Hkv={Hkv} splits={splits}")


def test_fp8_length_zero_and_one_exact():
    """len = 0 gives zeros; len = 1 gives v_scale times the E4M3 value of V[0], exactly."""
    case = W.fp8_contig_case(3, 8, 2, 128, 64, seq_lens=[0, 1, 64], seed=90, k_scale=0.5,
                             v_scale=0.25)
    out = DeviceCase(case).run_host()
    ref = oracle_out(case)
    assert np.all(out[0] == 0)
    assert np.array_equal(out[1].astype(np.float64), ref[1])
    compare(out, ref, "fp8 len 0/1")


def test_fp8_scales():
    """Scales that are not powers of two, large and small."""
    for ks, vs in ((0.37, 1.9), (3.0, 0.011), (1.0, 1.0)):
        case = W.fp8_contig_case(2, 16, 2, 128, 1000, seq_lens=[1000, 333], seed=91, k_scale=ks,
                                 v_scale=vs)
        compare(DeviceCase(case).run_host(), oracle_out(case), f"fp8 scales {ks} {vs}")


@pytest.mark.parametrize("ps", [16, 32, 64])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_fp8_paged(ps, D):
    say(f"[fp8] paged ps={ps} D={D}")
    case = W.fp8_paged_case(5, 16, 4, D, ps, 300, seq_lens=[1000, 1, 0, 457, 64], max_len=1024,
                            seed=92 + ps + D)
    dc = DeviceCase(case)
    ref = oracle_out(case)
    for splits in (0, 1, 7):
        compare(dc.run_host(splits), ref, f"fp8 paged ps={ps} D={D} splits={splits}")


def test_fp8_paged_equals_contiguous_bitwise(tune):
    """The same bytes through the paged and the contiguous layout give identical bits under the
    same plan.  By default a paged E4M3 cache at head_dim 128 takes 32-key tiles where the
    contiguous one takes 16, so the tile is pinned to 16 for the bitwise comparison; the
    default plans are checked against the oracle."""
    p = W.fp8_paged_case(3, 8, 2, 128, 32, 100, seq_lens=[700, 65, 1024], max_len=1024, seed=93)
    S_max = p.max_pages * p.page_size
    k = np.zeros((p.B, p.Hkv, S_max, p.D), np.uint8)
    v = np.zeros_like(k)
    for b in range(p.B):
        for i, page in enumerate(p.page_table[b]):
            if page < 0:
                continue
            k[b, :, i * p.page_size:(i + 1) * p.page_size] = p.k[page]
            v[b, :, i * p.page_size:(i + 1) * p.page_size] = p.v[page]
    c = W.Case("fp8_gathered", p.B, p.Hq, p.Hkv, p.D, p.scale, p.q, k, v, p.seq_lens, kv="fp8",
               k_scale=p.k_scale, v_scale=p.v_scale)
    ref = oracle_out(p)
    for splits in (0, 5):
        compare(DeviceCase(p).run_host(splits), ref, f"fp8 paged, default plan, splits={splits}")
        compare(DeviceCase(c).run_host(splits), ref, f"fp8 contiguous, default plan, splits={splits}")
    tune(tile_tokens=16)
    for splits in (0, 5):
        a = DeviceCase(p).run_host(splits)
        b = DeviceCase(c).run_host(splits)
        assert np.array_equal(_bits(a), _bits(b)), f"paged != contiguous (splits={splits})"


def test_fp8_matches_bf16_path_on_dequantised_cache():
    """With power-of-two scales the dequantised cache is exactly a bf16 cache; both GPU paths
    run the same contractions on the same values and agree to within rounding."""
    c = W.fp8_contig_case(2, 24, 4, 256, 2048, seq_lens=[2048, 999], seed=94, k_scale=0.5,
                          v_scale=0.25)
    table = np.array([0.0] * 256)
    grid = W._E4M3
    table[:127] = grid
    table[128:255] = -grid
    kd = W.f32_to_bf16_bits((table[c.k] * c.k_scale).astype(np.float32)).reshape(c.k.shape)
    vd = W.f32_to_bf16_bits((table[c.v] * c.v_scale).astype(np.float32)).reshape(c.v.shape)
    b = W.Case("dequantised", c.B, c.Hq, c.Hkv, c.D, c.scale, c.q, kd, vd, c.seq_lens)
    got, ref = DeviceCase(c).run_host(), DeviceCase(b).run_host()
    compare(got, ref.astype(np.float64), "fp8 vs bf16 path", atol=1e-5, rtol=1e-5)
    compare(got, oracle_out(c), "fp8 vs oracle")


def test_fp8_even_shares(tune):
    """Ragged E4M3 batches under several share counts (the even partition)."""
    case = W.fp8_contig_case(6, 16, 2, 128, 3000, seq_lens=[3000, 1, 0, 1500, 77, 2999], seed=95)
    dc = DeviceCase(case)
    ref = oracle_out(case)
    for shares in ("1", "7", "64", "1000"):
        for fold in (1, 2):
            tune(shares=int(shares), fold=fold, partition=2)
            compare(dc.run_host(), ref, f"fp8 even shares={shares} fold={fold}")


@pytest.mark.parametrize("paged,long_segments", [(False, False), (True, False), (False, True)])
def test_fp8_partials_then_combine_equals_one_call(paged, long_segments):
    """gqa_*_fp8_partials + gqa_decode_combine_fp8 on one stream give the one-call result bit for bit
    (the combine recomputes the E4M3 plan: paged tiles, the share rule of long segments)."""
    if paged:
        case = W.fp8_paged_case(4, 32, 8, 128, 32, 200, seq_lens=[1000, 1, 555, 1024], max_len=1024,
                                seed=96)
    elif long_segments:
        case = W.fp8_contig_case(4, 16, 2, 128, 4096, seq_lens=[4096, 4000, 3000, 4096], seed=98)
    else:
        case = W.fp8_contig_case(3, 24, 4, 256, 1500, seq_lens=[1500, 700, 3], seed=97, scale=1 / 16)
    dc = DeviceCase(case)
    cap, ps = case.capacity, case.page_size
    for splits in (0, 5):
        need = gd.gqa_decode_workspace_bytes(case.B, case.Hq, case.Hkv, case.D, cap, ps, splits)
        ws = gd.new_workspace(max(need, gd.COUNTER_BYTES))
        out = torch.empty((case.B, case.Hq, case.D), dtype=torch.float32, device="cuda")
        if paged:
            gd.gqa_paged_decode_fp8_partials(dc.q, dc.k, dc.v, dc.seq_lens, dc.page_table, case.scale,
                                             case.k_scale, case.v_scale, out=out, workspace=ws,
                                             num_splits=splits)
        else:
            gd.gqa_decode_fp8_partials(dc.q, dc.k, dc.v, dc.seq_lens, case.scale, case.k_scale,
                                       case.v_scale, out=out, workspace=ws, num_splits=splits)
        gd.gqa_decode_combine_fp8(ws, dc.seq_lens, out, case.B, case.Hq, case.Hkv, case.D, cap, ps,
                                  splits)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out.cpu().numpy()), _bits(dc.run_host(splits)))
