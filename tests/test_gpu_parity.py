"""HIP path against the CPU oracle, through the C ABI (needs an MI355X).

Tolerance (elementwise): |gpu - oracle| <= 2e-3 + 2e-3 |oracle|, the fp32
output against the fp64 oracle on unit-normal bf16 inputs.
"""
from __future__ import annotations

import dataclasses

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


# ------------------------------------------------------------------ the five workloads, full size
@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_workload_full_size(name):
    say(f"[parity] workload {name}: generating")
    case = W.make(name)
    dc = DeviceCase(case)
    plan = gd.gqa_decode_plan(case.B, case.Hq, case.Hkv, case.D, case.capacity, case.page_size)
    say(f"[parity] workload {name}: plan {plan.as_dict()}")
    outs = [dc.run_host() for _ in range(3)]
    say(f"[parity] workload {name}: oracle")
    ref = oracle_out(case)
    stats = compare(outs[0], ref, name)
    say(f"[parity] workload {name}: {stats}")
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32)), "not bit-exact across runs"


def test_million_key_context():
    """One sequence of 2^20 keys (256 MB of K and of V at head_dim 128), a length just short of
    the capacity: 32-bit buffer offsets up to 256 MB, 512 fixed splits of 2048 keys, against
    the oracle and bit-exact across runs."""
    S = 1 << 20
    say("[parity] 1M-key context: generating")
    rng = np.random.default_rng(75)

    def bf16_bits(shape):  # random sign, exponent 2^-4 .. 2^0, random mantissa: fast to draw
        return ((rng.integers(0, 2, shape, dtype=np.uint16) << 15)
                | (rng.integers(123, 128, shape, dtype=np.uint16) << 7)
                | rng.integers(0, 128, shape, dtype=np.uint16))

    case = W.Case("ctx_1m", 1, 8, 1, 128, W.default_scale(128), bf16_bits((1, 8, 128)),
                  bf16_bits((1, 1, S, 128)), bf16_bits((1, 1, S, 128)), np.array([S - 5], np.int32))
    dc = DeviceCase(case)
    plan = gd.gqa_decode_plan(1, 8, 1, 128, S)
    say(f"[parity] 1M-key context: plan {plan.as_dict()}")
    outs = [dc.run_host() for _ in range(2)]
    stats = compare(outs[0], oracle_out(case), "1M keys")
    say(f"[parity] 1M-key context: {stats}")
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


# ------------------------------------------------------------------ shape matrix
MATRIX = []
for D in (32, 64, 128, 256):
    for (Hq, Hkv) in ((8, 8), (8, 2), (12, 2), (16, 2), (16, 1)):
        MATRIX.append((D, Hq, Hkv))


@pytest.mark.parametrize("D,Hq,Hkv", MATRIX)
def test_matrix_ragged_with_nan_tail(D, Hq, Hkv):
    tt = {32: 64, 64: 64, 128: 32, 256: 16}[D]
    lens = [1, tt - 1, tt + 1, 3 * tt + 5, 517]
    S_max = 600
    say(f"[parity] matrix D={D} Hq={Hq} Hkv={Hkv} lens={lens}")
    case = W.contig_case(len(lens), Hq, Hkv, D, S_max, seq_lens=lens, seed=D + Hq + Hkv,
                         tail="nan")
    dc = DeviceCase(case)
    ref = oracle_out(case)
    for splits in (0, 1, 3):
        compare(dc.run_host(splits), ref, f"D={D} G={Hq // Hkv} splits={splits}")


@pytest.mark.parametrize("splits", [0, 1, 2, 7, 9, 64, 100, 10000])
def test_forced_split_counts(splits):
    say(f"[parity] forced splits {splits}")
    case = W.contig_case(2, 24, 4, 256, 2048, seq_lens=[2048, 1500], seed=21, scale=1 / 16)
    compare(DeviceCase(case).run_host(splits), oracle_out(case), f"splits={splits}")


def test_length_zero_and_one():
    say("[parity] len 0 / len 1")
    case = W.contig_case(3, 8, 2, 128, 64, seq_lens=[0, 1, 0], seed=22, tail="nan")
    dc = DeviceCase(case)
    for splits in (0, 1, 2):
        out = dc.run_host(splits)
        assert np.all(out[0] == 0) and np.all(out[2] == 0)
        v0 = W.bf16_bits_to_f32(case.v[1, :, 0, :]).reshape(2, 128)
        assert np.array_equal(out[1], np.repeat(v0, 4, axis=0)), "len 1 must return V[0] exactly"


def test_large_scores():
    say("[parity] large scores")
    case = W.contig_case(1, 8, 1, 128, 700, seed=23, scale=2.0)
    compare(DeviceCase(case).run_host(), oracle_out(case), "scale=2")


def test_peaky_small():
    say("[parity] peaky small")
    case = W.peaky_case(2, 16, 2, 128, 3000, frac=0.01, mul=8, seed=24)
    compare(DeviceCase(case).run_host(), oracle_out(case), "peaky")


def test_batch_zero():
    case = W.contig_case(1, 8, 2, 64, 16, seed=25)
    dc = DeviceCase(case)
    out = torch.empty((0, 8, 64), dtype=torch.float32, device="cuda")
    q0 = dc.q[:0]
    gd.gqa_decode(q0, dc.k[:0], dc.v[:0], dc.seq_lens[:0], case.scale, out=out)
    torch.cuda.synchronize()


def test_out_of_range_lengths_and_pages_are_clamped():
    """Device-resident values the host cannot check are clamped on the device, so no access
    leaves the caller's buffers: a negative length reads nothing (a zero row), a length past
    the capacity reads the capacity, and page ids outside [0, num_pages) read the nearest
    valid page.  The header leaves the output for such inputs unspecified; this checks the
    clamped result against the oracle on the clamped inputs, with an in-range sequence in
    the same batch, contiguous and paged, even shares and fixed splits."""
    say("[parity] clamped lengths and page ids")
    S = 512
    c = W.contig_case(3, 16, 4, 128, S, seq_lens=[100, 300, 200], seed=76)
    bad = c.seq_lens.copy()
    bad[0], bad[1] = -7, 10 ** 9
    c_bad = dataclasses.replace(c, seq_lens=bad)
    c_ref = dataclasses.replace(c, seq_lens=np.clip(bad, 0, S).astype(np.int32))
    ref = oracle_out(c_ref)
    for splits in (0, 3):
        compare(DeviceCase(c_bad).run_host(splits), ref, f"clamped lengths, splits={splits}")

    p = W.paged_case(3, 16, 4, 128, 32, 64, seq_lens=[512, 300, 200], max_len=S, seed=77)
    table = p.page_table.copy()
    table[0, 1], table[0, 5], table[1, 2] = -1, p.num_pages + 5, 1 << 30
    p_bad = dataclasses.replace(p, page_table=table)
    p_ref = dataclasses.replace(p, page_table=np.clip(table, 0, p.num_pages - 1).astype(np.int32))
    ref = oracle_out(p_ref)
    for splits in (0, 3):
        compare(DeviceCase(p_bad).run_host(splits), ref, f"clamped page ids, splits={splits}")


def test_side_stream_and_reused_workspace():
    say("[parity] side stream")
    case = W.contig_case(2, 8, 2, 128, 900, seq_lens=[900, 333], seed=26)
    dc = DeviceCase(case)
    ref = oracle_out(case)
    need = gd.gqa_decode_workspace_bytes(2, 8, 2, 128, 900, 0, 0)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        outs = [dc.run(0, workspace=ws, stream=s) for _ in range(2)]
    s.synchronize()
    for o in outs:
        compare(o.cpu().numpy(), ref, "side stream")


def test_side_stream_internal_buffers():
    """Kernels launched on stream s while the default stream is current, with no workspace or
    output passed: the binding allocates both for s, so blocks of the same size that the default
    stream allocates and fills (NaN bits) meanwhile never alias them while s is still busy."""
    say("[parity] side stream, internal buffers")
    case = W.contig_case(2, 8, 2, 128, 4096, seq_lens=[4096, 1333], seed=28)
    dc = DeviceCase(case)
    ref = oracle_out(case)
    need = gd.gqa_decode_workspace_bytes(2, 8, 2, 128, 4096, 0, 0)
    a = torch.randn(2048, 2048, device="cuda")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    outs = []
    for _ in range(4):
        with torch.cuda.stream(s):
            for _ in range(4):
                a = a @ a / 64  # keeps s busy, so the decode kernels are still queued below
        outs.append(dc.run(0, stream=s))
        junk = torch.empty(need, dtype=torch.uint8, device="cuda").fill_(255)
        junk_out = torch.empty((case.B, case.Hq, case.D), dtype=torch.float32, device="cuda").fill_(float("nan"))
        del junk, junk_out
    s.synchronize()
    torch.cuda.synchronize()
    for o in outs:
        compare(o.cpu().numpy(), ref, "side stream, internal buffers")


def test_binding_launches_on_the_current_stream():
    """The binding's current-stream query (torch's raw query where the build has it) names the
    stream torch considers current, outside and inside `torch.cuda.stream(s)`, and an explicit
    stream wins over it."""
    t = torch.empty(4, device="cuda")
    s = torch.cuda.Stream()
    assert gd._stream_ptr(None, t.device) == torch.cuda.current_stream().cuda_stream
    with torch.cuda.stream(s):
        assert gd._stream_ptr(None, t.device) == s.cuda_stream
    assert gd._stream_ptr(None, t.device) == torch.cuda.current_stream().cuda_stream
    assert gd._stream_ptr(s, t.device) == s.cuda_stream


def test_tuning_changed_by_another_thread_during_calls(tune):
    """One thread replaces the process-wide tuning over and over (plan partition, fold, combine
    kind) while another calls the library: each call copies the tuning once, so its split and
    combine launches always follow one plan, and every result matches the oracle."""
    import threading
    say("[parity] tuning changed during calls")
    case = W.contig_case(6, 32, 8, 128, 2048, seq_lens=[2048, 100, 0, 1500, 2047, 640], seed=96)
    dc = DeviceCase(case)
    ref = oracle_out(case)
    variants = [dict(partition=0, fold=0), dict(partition=1, fold=0), dict(partition=2, fold=2),
                dict(partition=1, combine=1), dict(partition=3, fold=0), dict(partition=2, fold=0)]
    need = 0
    for v in variants:
        with gd.tuning(**v):
            need = max(need, gd.gqa_decode_workspace_bytes(case.B, case.Hq, case.Hkv, case.D, case.capacity, 0, 0))
    ws = gd.new_workspace(max(need, gd.COUNTER_BYTES))
    base = gd.gqa_decode_get_tuning()
    stop = threading.Event()
    errors = []

    def flip():
        try:
            i = 0
            while not stop.is_set():
                t = gd.Tuning.from_buffer_copy(base)
                for k, val in variants[i % len(variants)].items():
                    setattr(t, k, val)
                gd.gqa_decode_set_tuning(t)
                i += 1
        except Exception as e:  # reported on the main thread
            errors.append(repr(e))

    th = threading.Thread(target=flip)
    th.start()
    try:
        outs = [dc.run(0, workspace=ws) for _ in range(60)]
        torch.cuda.synchronize()
    finally:
        stop.set()
        th.join(timeout=30)
        gd.gqa_decode_set_tuning(base)
    assert not errors, errors
    for o in outs:
        compare(o.cpu().numpy(), ref, "tuning changed during calls")


def test_concurrent_host_threads():
    """Four host threads call the library at once (ctypes drops the GIL for the call), each on
    its own stream with its own workspace and outputs, one plan kind per thread: the small-job
    in-kernel fold, fixed splits, even shares and a paged cache. Every result equals the same call
    made alone, bit for bit, and that call matches the oracle."""
    import threading
    say("[parity] concurrent host threads")
    cases = [W.make("tiny_gqa4_d64_ctx512"),
             W.contig_case(1, 24, 4, 256, 2048, seed=93, name="fixed"),
             W.contig_case(12, 32, 4, 128, 3000, seq_lens=[3000, 17, 2500, 0, 999, 3000, 1, 2048,
                                                           640, 2999, 1500, 33], seed=94, name="even"),
             W.paged_case(6, 16, 4, 128, 32, 400, seq_lens=[1, 700, 2048, 31, 1200, 999], max_len=2048,
                          seed=95, name="paged")]
    dcs = [DeviceCase(c) for c in cases]
    alone = []
    for c, dc in zip(cases, dcs):
        o = dc.run_host()
        compare(o, oracle_out(c), f"concurrent threads, alone: {c.name}")
        alone.append(o)
    torch.cuda.synchronize()
    calls = 25
    results = [None] * len(cases)
    errors = []

    def work(i):
        try:
            c, dc = cases[i], dcs[i]
            need = gd.gqa_decode_workspace_bytes(c.B, c.Hq, c.Hkv, c.D, c.capacity, c.page_size, 0)
            s = torch.cuda.Stream()
            ws = gd.new_workspace(max(need, gd.COUNTER_BYTES), stream=s)  # zeroed on s
            with torch.cuda.stream(s):
                outs = [torch.empty((c.B, c.Hq, c.D), dtype=torch.float32, device="cuda") for _ in range(calls)]
            for o in outs:
                dc.run(0, out=o, workspace=ws, stream=s)
            s.synchronize()
            results[i] = [o.cpu().numpy() for o in outs]
        except Exception as e:  # reported on the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a host thread did not finish"
    assert not errors, errors
    for i, c in enumerate(cases):
        for o in results[i]:
            assert np.array_equal(o.view(np.uint32), alone[i].view(np.uint32)), f"{c.name}: differs from the call alone"


# ------------------------------------------------------------------ paged
@pytest.mark.parametrize("ps", [16, 32, 64, 48])
@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_paged_matrix(ps, D):
    say(f"[parity] paged ps={ps} D={D}")
    lens = [1, ps - 1, ps, ps + 1, 5 * ps + 3, 700]
    case = W.paged_case(len(lens), 16, 4, D, ps, 200, seq_lens=lens, max_len=704, seed=ps + D)
    dc = DeviceCase(case)
    ref = oracle_out(case)
    # 100 splits (clamped to the tile count): one tile per wave, the lock-step path
    for splits in (0, 1, 5, 100):
        compare(dc.run_host(splits), ref, f"paged ps={ps} D={D} splits={splits}")


@pytest.mark.parametrize("ps", [256, 1024, 208])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_large_pages(ps, kv):
    """Pages far longer than a tile (many tiles per page, one page-table entry serving them all)
    and a page size that is no power of two: ragged lengths on both sides of page boundaries,
    fixed splits, even shares and one tile per wave."""
    say(f"[parity] large pages ps={ps} kv={kv}")
    lens = [1, ps - 1, ps, ps + 1, 3 * ps + 17, 0, 2 * ps - 5]
    max_len = 4 * ps
    pages = sum((n + ps - 1) // ps for n in lens) + 2
    make = W.paged_case if kv == "bf16" else W.fp8_paged_case
    case = make(len(lens), 16, 4, 128, ps, pages, seq_lens=lens, max_len=max_len, seed=ps + (kv == "fp8"))
    dc = DeviceCase(case)
    ref = oracle_out(case)
    for splits in (0, 1, 7, 1000):
        compare(dc.run_host(splits), ref, f"ps={ps} {kv} splits={splits}")


def test_paged_equals_contiguous_bitwise(tune):
    """Pages holding the same rows as a contiguous cache give the same bits (same plan)."""
    say("[parity] paged == contiguous")
    B, Hq, Hkv, D, ps, S = 3, 32, 8, 128, 32, 1024
    c = W.contig_case(B, Hq, Hkv, D, S, seq_lens=[1024, 77, 500], seed=27)
    pages = S // ps
    k_pool = np.zeros((B * pages, Hkv, ps, D), np.uint16)
    v_pool = np.zeros_like(k_pool)
    table = np.zeros((B, pages), np.int32)
    for b in range(B):
        for i in range(pages):
            pg = b * pages + i
            k_pool[pg] = c.k[b, :, i * ps:(i + 1) * ps]
            v_pool[pg] = c.v[b, :, i * ps:(i + 1) * ps]
            table[b, i] = pg
    p = W.Case("paged_copy", B, Hq, Hkv, D, c.scale, c.q, k_pool, v_pool, c.seq_lens, table, ps)
    # the plan's one-tile-per-wave splits (a small job); fixed splits of several tiles; one tile
    # per wave (64 splits of 16 keys); then even shares
    for splits in (0, 7, 64):
        a = DeviceCase(c).run_host(splits)
        b = DeviceCase(p).run_host(splits)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"splits={splits}"
    tune(partition=2)
    a = DeviceCase(c).run_host()
    b = DeviceCase(p).run_host()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "even shares"


def test_paged_page_permutation_bitwise():
    say("[parity] page permutation")
    p = W.paged_case(4, 32, 8, 128, 32, 300, seq_lens=[2000, 31, 1000, 33], max_len=2048,
                     seed=28)
    rng = np.random.default_rng(6)
    perm = rng.permutation(p.num_pages)
    k2 = np.empty_like(p.k)
    v2 = np.empty_like(p.v)
    k2[perm] = p.k
    v2[perm] = p.v
    t2 = np.where(p.page_table >= 0, perm[np.maximum(p.page_table, 0)], -1).astype(np.int32)
    q = W.Case("perm", p.B, p.Hq, p.Hkv, p.D, p.scale, p.q, k2, v2, p.seq_lens, t2, p.page_size)
    a = DeviceCase(p).run_host()
    b = DeviceCase(q).run_host()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    compare(a, oracle_out(p), "paged permutation")


# ------------------------------------------------------------------ workspace reuse and call variants
@pytest.mark.parametrize("fold", [0, 2], ids=["default", "fused"])
def test_shared_workspace_across_plans(tune, fold):
    """One workspace whose partial region was never initialised (all bytes 0xFF: NaN floats;
    only the arrival counters are zero) serves calls with different shapes and plans (even
    shares, fixed splits, folded in a combine kernel or in the split kernel) back to back."""
    say(f"[parity] shared workspace fold={fold}")
    tune(fold=fold)
    a = W.contig_case(1, 8, 1, 128, 20000, seed=30)          # one long sequence, fixed splits
    b = W.contig_case(3, 16, 4, 64, 700, seq_lens=[700, 5, 300], seed=31)
    c = W.paged_case(4, 32, 8, 128, 32, 300, seq_lens=[1000, 0, 555, 1024], max_len=1024, seed=32)
    ws = torch.full((1 << 24,), 255, dtype=torch.uint8, device="cuda")
    ws[:gd.COUNTER_BYTES] = 0  # only the arrival counters must start at zero
    da, db, dc = DeviceCase(a), DeviceCase(b), DeviceCase(c)
    ra, rb, rc = oracle_out(a), oracle_out(b), oracle_out(c)
    for _ in range(3):
        oa = da.run(0, workspace=ws)
        ob = db.run(3, workspace=ws)
        oc = dc.run(0, workspace=ws)
        od = da.run(37, workspace=ws)
        torch.cuda.synchronize()
        compare(oa.cpu().numpy(), ra, "plan A")
        compare(ob.cpu().numpy(), rb, "plan B, 3 splits")
        compare(oc.cpu().numpy(), rc, "plan C, paged even shares")
        compare(od.cpu().numpy(), ra, "plan A, 37 splits")


@pytest.mark.parametrize("mode", ["default", "tree"])
def test_combine_thread_per_column(tune, mode):
    """Plans with few pieces per segment at full length use one thread per output column
    (default); the tuning's combine = 1 forces the tree.  Both match the oracle and are
    bit-exact across runs: even shares whose short sequences make the long ones span more
    than 16 shares (several rounds of loads per thread), paged shares, a few fixed splits,
    and multi-query rows."""
    say(f"[parity] combine {mode}")
    if mode == "tree":
        tune(combine=1)
    lens = [4096, 3, 0, 17, 1, 2000] + [1] * 10
    cases = [
        (W.contig_case(16, 16, 4, 128, 4096, seq_lens=lens, seed=62), 0),
        (W.paged_case(16, 32, 8, 128, 32, 3000, max_len=4096, seed=63), 0),
        (W.contig_case(3, 24, 4, 256, 1500, seq_lens=[1500, 700, 3], seed=64, scale=1 / 16), 5),
        (W.mq_case(16, 2, 16, 4, 128, 3000, seq_lens=[3000, 4, 0, 999, 1500, 2] + [2500] * 10, seed=65), 0),
    ]
    for case, splits in cases:
        dc = DeviceCase(case)
        runs = [dc.run_host(splits) for _ in range(2)]
        compare(runs[0], oracle_out(case), f"{mode} {case.name} splits={splits}")
        assert np.array_equal(runs[0].view(np.uint32), runs[1].view(np.uint32))


@pytest.mark.parametrize("cols", ["2", "4", "8", "16"])
def test_combine_column_widths(tune, cols):
    """Every combine width (lanes of a column merged by row rotations, row-pair and
    half-wave swaps, then the waves) matches the oracle and is bit-exact across runs,
    for fixed splits (several rounds of loads per thread) and ragged even shares."""
    say(f"[parity] combine columns={cols}")
    tune(combine_cols=int(cols), fold=1)  # the tree combine runs in its own kernel
    fixed = W.contig_case(2, 24, 4, 256, 3000, seq_lens=[3000, 1111], seed=60, scale=1 / 16)
    even = W.paged_case(5, 16, 4, 128, 32, 400, seq_lens=[2048, 1, 0, 777, 1500], max_len=2048, seed=61)
    for case, splits in ((fixed, 0), (fixed, 150), (even, 0)):
        dc = DeviceCase(case)
        runs = [dc.run_host(splits) for _ in range(2)]
        compare(runs[0], oracle_out(case), f"columns={cols} splits={splits}")
        assert np.array_equal(runs[0].view(np.uint32), runs[1].view(np.uint32))


@pytest.mark.parametrize("pv", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_pv_modes(tune, pv, D):
    """Both PV contractions (fp32 MFMA; bf16 MFMA with P split hi+lo) match the oracle,
    with a NaN-poisoned tail and ragged lengths."""
    say(f"[parity] pv={pv} D={D}")
    tune(pv_mode=0 if pv == "f32" else 1)
    assert gd.gqa_decode_plan(2, 16, 2, D, 300).pv_mode == (0 if pv == "f32" else 1)
    case = W.contig_case(3, 16, 2, D, 300, seq_lens=[300, 17, 129], seed=40 + D, tail="nan")
    dc = DeviceCase(case)
    ref = oracle_out(case)
    for splits in (0, 1, 4):
        compare(dc.run_host(splits), ref, f"pv={pv} D={D} splits={splits}")
    pk = W.peaky_case(1, 8, 1, D, 4000, frac=0.01, mul=8, seed=41)
    compare(DeviceCase(pk).run_host(), oracle_out(pk), f"peaky pv={pv} D={D}")


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("long_segments", [False, True])
def test_partials_then_combine_equals_one_call(paged, long_segments):
    """gqa_*_partials + gqa_decode_combine on one stream give the one-call result bit for bit
    (long contiguous segments: with one share per CU in both kernels)."""
    say(f"[parity] partials + combine, paged={paged} long={long_segments}")
    if paged:
        case = W.paged_case(4, 32, 8, 128, 32, 200, seq_lens=[1000, 1, 555, 1024], max_len=1024,
                            seed=50)
    elif long_segments:
        case = W.contig_case(4, 16, 2, 128, 4096, seq_lens=[4096, 4000, 3000, 4096], seed=52)
    else:
        case = W.contig_case(3, 24, 4, 256, 1500, seq_lens=[1500, 700, 3], seed=51, scale=1 / 16)
    dc = DeviceCase(case)
    one = dc.run_host()
    cap, ps = case.capacity, case.page_size
    for splits in (0, 5):
        need = gd.gqa_decode_workspace_bytes(case.B, case.Hq, case.Hkv, case.D, cap, ps, splits)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
        out = torch.empty((case.B, case.Hq, case.D), dtype=torch.float32, device="cuda")
        if paged:
            gd.gqa_paged_decode_partials(dc.q, dc.k, dc.v, dc.seq_lens, dc.page_table, case.scale,
                                         out=out, workspace=ws, num_splits=splits)
        else:
            gd.gqa_decode_partials(dc.q, dc.k, dc.v, dc.seq_lens, case.scale, out=out, workspace=ws,
                                   num_splits=splits)
        gd.gqa_decode_combine(ws, dc.seq_lens, out, case.B, case.Hq, case.Hkv, case.D, cap, ps,
                              splits)
        torch.cuda.synchronize()
        two = out.cpu().numpy()
        ref = dc.run_host(splits)
        assert np.array_equal(two.view(np.uint32), ref.view(np.uint32))
    compare(one, oracle_out(case), "partials+combine")


# ------------------------------------------------------------------ even-share partition
EVEN_LENS = {
    "mixed": [1, 0, 700, 3, 5000, 17, 0, 2048, 1, 33],
    "short_many": [(7 * i) % 40 for i in range(100)],          # B > 64: the scan loops over chunks
    "one_long": [0, 0, 20000, 0],
    "all_zero": [0, 0, 0],
}


@pytest.mark.parametrize("lens", list(EVEN_LENS))
@pytest.mark.parametrize("shares", ["1", "3", "7", "64", "1000"])
@pytest.mark.parametrize("fold", [1, 2], ids=["kernel", "fused"])
def test_even_shares_contiguous(tune, lens, shares, fold):
    """Equal shares of the concatenated tiles, any share count, ragged and empty sequences
    (the even partition asked for, with a capacity of at least 1024 keys so that short cases
    take it too), folded by the combine kernel and in the split kernel."""
    say(f"[parity] even shares={shares} lens={lens} fold={fold}")
    tune(shares=int(shares), fold=fold, partition=2)
    L = EVEN_LENS[lens]
    S_max = max(max(L), 1024)
    case = W.contig_case(len(L), 16, 4, 128, S_max, seq_lens=L, seed=60, tail="nan")
    p = gd.gqa_decode_plan(case.B, 16, 4, 128, S_max)
    assert p.partition == 1 and p.fused == (fold == 2)
    dc = DeviceCase(case)
    out = [dc.run_host() for _ in range(2)]
    compare(out[0], oracle_out(case), f"even shares={shares} {lens}")
    assert np.array_equal(out[0].view(np.uint32), out[1].view(np.uint32))
    for b, n in enumerate(L):
        if n == 0:
            assert np.all(out[0][b] == 0)


@pytest.mark.parametrize("shares", ["5", "0"])
@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_even_shares_paged(tune, shares, D):
    say(f"[parity] even shares paged D={D} shares={shares}")
    tune(shares=int(shares), partition=2)
    L = [1, 0, 900, 31, 2000, 16, 0, 1500]
    case = W.paged_case(len(L), 8, 2, D, 32, 250, seq_lens=L, max_len=2048, seed=61 + D)
    assert gd.gqa_decode_plan(case.B, 8, 2, D, 2048, 32).partition == 1
    compare(DeviceCase(case).run_host(), oracle_out(case), f"even paged D={D}")


def test_fixed_and_even_agree_with_oracle(tune):
    say("[parity] fixed vs even")
    case = W.paged_case(8, 32, 8, 128, 32, 2100, max_len=8192, seed=62)
    dc = DeviceCase(case)
    ref = oracle_out(case)
    even = dc.run_host()
    tune(partition=1)
    fixed = dc.run_host()
    compare(even, ref, "even")
    compare(fixed, ref, "fixed")


@pytest.mark.parametrize("halve", ["default", "0"])
def test_even_shares_long_segments(tune, halve):
    """Contiguous batches whose segments average >= 128 tiles take one share per CU (half the
    launched shares; the rest exit); shorter ones keep two.  Both sides of the rule, with the
    rule switched off, and the many-sequence walk (B > 64), against the oracle and bit-exact
    across runs."""
    say(f"[parity] long segments, halve={halve}")
    if halve == "0":
        tune(halve_long=0)
    rng = np.random.default_rng(70)
    cases = [
        W.contig_case(8, 32, 4, 128, 4096, seq_lens=[4096, 4000, 2048, 3000, 4096, 1, 0, 4095], seed=71),
        W.contig_case(8, 32, 4, 128, 4096, seq_lens=[100, 4, 0, 300, 17, 1000, 2, 64], seed=72),
        W.contig_case(70, 16, 2, 128, 2304, seq_lens=rng.integers(2048, 2305, 70), seed=73),
        W.mq_case(8, 2, 16, 4, 128, 4096, seq_lens=[4096, 2048, 3000, 4096, 2500, 4096, 2200, 3333], seed=74),
    ]
    for case in cases:
        dc = DeviceCase(case)
        runs = [dc.run_host() for _ in range(2)]
        compare(runs[0], oracle_out(case), f"{case.name} halve={halve}")
        assert np.array_equal(runs[0].view(np.uint32), runs[1].view(np.uint32))


@pytest.mark.parametrize("nt", ["0", "1"])
def test_cache_policy_variants(tune, nt):
    """Both K/V load cache policies give the same bits (only the hint differs)."""
    say(f"[parity] streaming={nt}")
    case = W.contig_case(2, 16, 2, 128, 3000, seq_lens=[3000, 1234], seed=70, tail="nan")
    dc = DeviceCase(case)
    base = dc.run_host()
    tune(streaming=int(nt))
    assert gd.gqa_decode_plan(2, 16, 2, 128, 3000).streaming == int(nt)  # default: 1
    out = dc.run_host()
    assert np.array_equal(out.view(np.uint32), base.view(np.uint32))
    compare(out, oracle_out(case), f"nt={nt}")


# ------------------------------------------------------------------ proportional splits (partition = 3)
def _prop_cases():
    """Factories (each test builds only its own case)."""
    lens70 = np.random.default_rng(190).integers(0, 2305, 70)
    return [
        lambda: W.contig_case(10, 16, 4, 128, 5000, seq_lens=[1, 0, 700, 3, 5000, 17, 0, 2048, 1, 33], seed=191, tail="nan"),
        lambda: W.paged_case(16, 32, 8, 128, 32, 4000, max_len=8192, seed=192),
        lambda: W.contig_case(70, 16, 2, 128, 2304, seq_lens=lens70, seed=193),
        lambda: W.contig_case(100, 16, 4, 128, 1024, seq_lens=[(7 * i) % 40 for i in range(100)], seed=194),
        lambda: W.contig_case(3, 16, 4, 128, 1024, seq_lens=[0, 0, 0], seed=195),
        lambda: W.contig_case(4, 32, 4, 128, 20000, seq_lens=[0, 0, 20000, 0], seed=196),
        lambda: W.contig_case(8, 32, 4, 128, 4096, seed=197),
        lambda: W.mq_case(12, 3, 16, 4, 128, 3000, seq_lens=[3000, 2, 0, 999, 1500, 2500] * 2, seed=198),
        lambda: W.fp8_contig_case(18, 16, 2, 128, 3000, seq_lens=[3000, 1, 0, 1500, 77, 2999] * 3, seed=199),
        lambda: W.fp8_paged_case(10, 16, 4, 128, 32, 400, seq_lens=[2048, 1, 0, 777, 1500] * 2, max_len=2048, seed=200),
        lambda: W.paged_case(6, 8, 2, 64, 48, 300, seq_lens=[1, 2000, 47, 49, 0, 1500], max_len=2400, seed=201),
        lambda: W.contig_case(2, 24, 4, 256, 4096, seq_lens=[4096, 3001], seed=202, scale=1 / 16),
    ]


_PROP_REF = {}
_PROP_CASE = {}


@pytest.mark.parametrize("shares", ["0", "7", "1000"])
@pytest.mark.parametrize("i", range(12))
def test_proportional_splits(tune, i, shares):
    """Proportional splits: each (sequence, kv head) segment cut into ceil(n / L) equal splits,
    one piece per workgroup, folded by the thread-per-column combine -- ragged lengths with zeros
    and NaN tails, paged (page 32 and 48), more than 64 sequences, all sequences empty, one long
    sequence among empty ones, uniform lengths, multi-query rows, E4M3, head_dim 64 and 256,
    several share counts; against the oracle and bit-exact across runs."""
    tune(partition=3, shares=int(shares))
    if i not in _PROP_CASE:
        _PROP_CASE.clear()   # one case held at a time (the share counts of one case run together or not)
        _PROP_CASE[i] = _prop_cases()[i]()
    case = _PROP_CASE[i]
    say(f"[parity] proportional splits {case.name} B={case.B} shares={shares}")
    plan_fn = gd.gqa_decode_plan_fp8 if case.kv == "fp8" else gd.gqa_decode_plan
    p = plan_fn(case.B, case.M * case.Hq, case.Hkv, case.D, case.capacity, case.page_size)
    assert p.partition == 2, p.as_dict()
    dc = DeviceCase(case)
    a = dc.run_host()
    if i not in _PROP_REF:
        _PROP_REF[i] = oracle_out(case)
    compare(a, _PROP_REF[i], f"proportional {case.name} shares={shares}")
    assert np.array_equal(np.ascontiguousarray(a).view(np.uint32), np.ascontiguousarray(dc.run_host()).view(np.uint32))
    lens = np.asarray(case.seq_lens)
    if case.M == 1:
        assert np.all(a[lens == 0] == 0)


# ------------------------------------------------------------------ very large batches
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
def test_very_large_batch(paged):
    """Thousands of short ragged sequences (zeros included): the even shares' length scan runs
    over dozens of 64-sequence chunks before a share knows its first segment."""
    rng = np.random.default_rng(180 + paged)
    B = 1000 if paged else 2000
    lens = rng.integers(0, 301, B)
    lens[rng.random(B) < 0.1] = 0
    say(f"[parity] very large batch B={B} paged={paged}")
    if paged:
        case = W.paged_case(B, 8, 2, 128, 32, int(sum((n + 31) // 32 for n in lens)) + 5, seq_lens=lens,
                            max_len=512, seed=182)
    else:
        case = W.contig_case(B, 8, 2, 128, 512, seq_lens=lens, seed=183, tail="nan")
    p = gd.gqa_decode_plan(case.B, case.Hq, case.Hkv, case.D, case.capacity, case.page_size)
    assert p.partition == 1, p.as_dict()
    dc = DeviceCase(case)
    a = dc.run_host()
    compare(a, oracle_out(case), f"very large batch B={B} paged={paged}")
    assert np.array_equal(a.view(np.uint32), dc.run_host().view(np.uint32))
    assert np.all(a[lens == 0] == 0)


def test_multi_head_attention_shape():
    """G = 1 (16 kv heads, one query head each) over fixed splits and even shares."""
    say("[parity] G = 1")
    case = W.contig_case(5, 16, 16, 128, 3000, seq_lens=[3000, 1, 0, 1777, 2999], seed=184, tail="nan")
    dc = DeviceCase(case)
    ref = oracle_out(case)
    for splits in (0, 1, 9):
        compare(dc.run_host(splits), ref, f"G=1 splits={splits}")


# ------------------------------------------------------------------ small jobs: fixed splits of one 16-key tile per wave
def _small_job_cases():
    return [
        lambda: W.contig_case(2, 16, 4, 128, 1024, seq_lens=[1024, 333], seed=160, tail="nan"),
        lambda: W.contig_case(3, 8, 2, 64, 700, seq_lens=[700, 300, 5], seed=161, tail="nan"),
        lambda: W.contig_case(8, 8, 1, 256, 512, seq_lens=[512, 0, 1, 17, 500, 64, 65, 333], seed=162, scale=1 / 16),
        lambda: W.contig_case(8, 32, 8, 128, 1024, seq_lens=[1024, 3, 0, 999, 512, 1000, 64, 777], seed=163),   # 1024 workgroups
        lambda: W.contig_case(2, 8, 2, 32, 4096, seq_lens=[4096, 4000], seed=164),
        lambda: W.paged_case(4, 8, 2, 128, 32, 100, seq_lens=[1024, 300, 700, 9], max_len=1024, seed=165),
        lambda: W.paged_case(2, 32, 8, 64, 16, 80, seq_lens=[512, 400], max_len=512, seed=166),
        lambda: W.fp8_contig_case(2, 16, 4, 128, 1024, seq_lens=[1024, 77], seed=167),
        lambda: W.fp8_paged_case(4, 8, 2, 128, 32, 100, seq_lens=[1024, 300, 700, 9], max_len=1024, seed=168),
        lambda: W.mq_case(3, 4, 16, 4, 128, 1024, seq_lens=[1024, 4, 600], seed=169, tail="nan"),
        lambda: W.mq_paged_case(2, 2, 16, 4, 128, 32, 80, [1000, 33], max_len=1024, seed=170),
    ]


@pytest.mark.parametrize("i", range(11))
def test_small_job_plans(i):
    """Batches small enough that one 16-key tile per wave in fixed splits takes at most four
    workgroups per CU (contiguous, paged, E4M3, multi-query; ragged lengths, zeros, NaN tails):
    the plan is those splits, the result matches the oracle and is bit-exact across runs."""
    case = _small_job_cases()[i]()
    say(f"[parity] small job {case.name} B={case.B} Hkv={case.Hkv} D={case.D} cap={case.capacity}")
    plan_fn = gd.gqa_decode_plan_fp8 if case.kv == "fp8" else gd.gqa_decode_plan
    p = plan_fn(case.B, case.M * case.Hq, case.Hkv, case.D, case.capacity, case.page_size)
    assert p.partition == 0 and p.tile_tokens == 16 and p.split_tokens == 64, p.as_dict()
    dc = DeviceCase(case)
    a = dc.run_host()
    compare(a, oracle_out(case), f"small job {case.name}")
    assert np.array_equal(np.ascontiguousarray(a).view(np.uint32), np.ascontiguousarray(dc.run_host()).view(np.uint32))


# ------------------------------------------------------------------ tile size and register buffering (A/B variants)
@pytest.mark.parametrize("dbuf", [0, 1])
@pytest.mark.parametrize("tile", [16, 32, 64])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_tile_and_buffer_variants(tune, tile, dbuf, D):
    """Keys per wave tile 16, 32 or 64 (where K+V of a tile fit 16 KB per wave) with one or two
    register tiles per wave, against the oracle: ragged lengths with a NaN tail over fixed splits
    (one-tile and key-range workgroups) and even shares, and a paged cache whose page holds 32
    keys (the tile is halved until it divides the page)."""
    tune(tile_tokens=tile, double_buffer=dbuf)
    say(f"[parity] tile={tile} dbuf={dbuf} D={D}")
    lens = [1, 15, 17, 53, 700, 2000]
    case = W.contig_case(len(lens), 16, 2, D, 2048, seq_lens=lens, seed=150 + D + tile + dbuf, tail="nan")
    plan = gd.gqa_decode_plan(case.B, 16, 2, D, 2048)
    assert plan.double_buffer == dbuf
    assert plan.tile_tokens == (tile if tile * D * 4 <= 16384 else plan.tile_tokens)
    dc = DeviceCase(case)
    ref = oracle_out(case)
    for splits in (0, 1, 3, 40):
        a = dc.run_host(splits)
        compare(a, ref, f"tile={tile} dbuf={dbuf} D={D} splits={splits}")
        assert np.array_equal(a.view(np.uint32), dc.run_host(splits).view(np.uint32))
    paged = W.paged_case(4, 16, 2, D, 32, 300, seq_lens=[1, 900, 2048, 333], max_len=2048, seed=151 + D)
    compare(DeviceCase(paged).run_host(), oracle_out(paged), f"tile={tile} dbuf={dbuf} paged D={D}")


@pytest.mark.parametrize("name,fields", [
    ("batched_gqa8_d128_ctx16k", {"tile_tokens": 32}),
    ("batched_gqa8_d128_ctx16k", {"double_buffer": 1}),
    ("paged_gqa4_d128_ragged8k", {"tile_tokens": 32}),
    ("paged_gqa4_d128_ragged8k", {"double_buffer": 1}),
    ("paged_gqa4_d128_ragged8k", {"shares": 256, "double_buffer": 1}),
    ("long_gqa8_d128_ctx128k_peaky", {"tile_tokens": 32}),
    ("long_gqa8_d128_ctx128k_peaky", {"double_buffer": 1}),
    ("batched_gqa8_d128_ctx16k", {"partition": 3}),
    ("paged_gqa4_d128_ragged8k", {"partition": 3}),
    ("gqa6_d256_ctx4096", {"partition": 3}),
    ("long_gqa8_d128_ctx128k_peaky", {"partition": 3}),
], ids=lambda x: x if isinstance(x, str) else ",".join(f"{k}={v}" for k, v in x.items()))
def test_variant_workloads(tune, name, fields):
    """The full-size workloads under the tile and buffering variants that bench.py --ab times."""
    tune(**fields)
    say(f"[parity] variant {fields} workload {name}")
    case = W.make(name)
    compare(DeviceCase(case).run_host(), oracle_out(case), f"{fields} {name}")


# ------------------------------------------------------------------ QK^T on the vector ALU (A/B variant)
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 2), (12, 2), (16, 2), (16, 1), (24, 4)])
def test_qk_valu_variant(tune, D, Hq, Hkv):
    """The vector-ALU QK^T (v_dot2c over each lane's head-dim quarter, lane swaps, an LDS
    transpose) against the oracle, with ragged lengths and a NaN tail, in fixed splits (one-tile
    and key-range workgroups) and even shares, contiguous and paged; bit-exact across runs."""
    tune(qk_mode=1)
    say(f"[parity] qk valu D={D} Hq={Hq} Hkv={Hkv}")
    lens = [1, 15, 17, 53, 700, 2000]
    case = W.contig_case(len(lens), Hq, Hkv, D, 2048, seq_lens=lens, seed=130 + D + Hq, tail="nan")
    assert gd.gqa_decode_plan(case.B, Hq, Hkv, D, 2048).qk_mode == 1
    dc = DeviceCase(case)
    ref = oracle_out(case)
    for splits in (0, 1, 3, 40):
        a = dc.run_host(splits)
        compare(a, ref, f"qk valu D={D} G={Hq // Hkv} splits={splits}")
        assert np.array_equal(a.view(np.uint32), dc.run_host(splits).view(np.uint32))
    paged = W.paged_case(4, Hq, Hkv, D, 32, 300, seq_lens=[1, 900, 2048, 333], max_len=2048, seed=131 + D)
    compare(DeviceCase(paged).run_host(), oracle_out(paged), f"qk valu paged D={D}")


@pytest.mark.parametrize("name", ["gqa6_d256_ctx4096", "batched_gqa8_d128_ctx16k", "paged_gqa4_d128_ragged8k",
                                  "long_gqa8_d128_ctx128k_peaky"])
def test_qk_valu_workloads(tune, name):
    tune(qk_mode=1)
    say(f"[parity] qk valu workload {name}")
    case = W.make(name)
    assert gd.gqa_decode_plan(case.B, case.Hq, case.Hkv, case.D, case.capacity, case.page_size).qk_mode == 1
    compare(DeviceCase(case).run_host(), oracle_out(case), f"qk valu {name}")
