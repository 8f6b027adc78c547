"""Host-side logic of the C-ABI library, on the CPU (no kernel is launched)."""
import ctypes
import os
import re

import pytest

import decode_attention_04_amd as gd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_decode.h")

WORKLOAD_SHAPES = [  # (B, Hq, Hkv, D, capacity, page_size)
    (1, 8, 2, 64, 512, 0),
    (1, 24, 4, 256, 4096, 0),
    (16, 32, 4, 128, 16384, 0),
    (32, 32, 8, 128, 8192, 32),
    (1, 8, 1, 128, 131072, 0),
]


@pytest.fixture(scope="module")
def lib():
    return gd.load()


def expected_workspace(B, Hq, Hkv, D, p):
    """The arrival counters' header, then partial blocks (slots) of G x (D + 2) floats, each
    region rounded up to 256 bytes."""
    if p.direct:
        return 0
    align = lambda x: (x + 255) // 256 * 256
    G = Hq // Hkv
    return gd.COUNTER_BYTES + align(p.slots * G * D * 4) + align(p.slots * G * 2 * 4)


def tree_nodes(S, F):
    """Nodes above the leaves of a fold tree over S partials with fan-in F (written out)."""
    nodes, n = 0, S
    while n > 1:
        n = -(-n // F)
        nodes += n
    return nodes


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_\w+)\s*\(", text)))


def test_header_declares_what_the_binding_exports():
    assert declared_functions() == sorted(gd.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(8):
        assert lib.gqa_status_string(code)
    assert b"unknown" in lib.gqa_status_string(99)


@pytest.mark.parametrize("shape", WORKLOAD_SHAPES)
@pytest.mark.parametrize("cu", [256, 304, 80, 1])
def test_plan_invariants(shape, cu):
    B, Hq, Hkv, D, cap, ps = shape
    p = gd.gqa_decode_plan(B, Hq, Hkv, D, cap, ps, 0, cu)
    assert p.tile_tokens % 16 == 0
    if ps:
        assert ps % p.tile_tokens == 0        # one page-table lookup per tile
    tiles = -(-cap // p.tile_tokens)
    if p.partition == 1:                      # even shares
        assert p.num_splits == 0 and p.direct == 0
        assert 1 <= p.grid <= 2 * cu
        assert p.grid * 4 <= B * Hkv * tiles + 3   # at least one tile per wave at full length
        assert p.slots == p.grid + B * Hkv
        assert p.split_tokens % p.tile_tokens == 0
        assert p.split_tokens * p.grid >= B * Hkv * cap
        # by default a combine kernel folds the pieces; with the tuning's fold = 2 the split
        # kernel does, one counter per segment
        assert p.fused == 0 and p.counters == 0 and p.fold_fanin == 0
        with gd.tuning(fold=2):
            f = gd.gqa_decode_plan(B, Hq, Hkv, D, cap, ps, 0, cu)
            assert f.fused == 1 and f.counters == B * Hkv and f.slots == p.slots
    else:                                      # fixed splits
        assert p.split_tokens % p.tile_tokens == 0
        assert p.num_splits * p.split_tokens >= cap
        assert (p.num_splits - 1) * p.split_tokens < cap  # no split starts past the capacity
        assert p.grid == B * Hkv * p.num_splits
        assert p.direct == (p.num_splits == 1)
        assert p.slots == B * Hkv * p.num_splits
        # fixed splits fold in the split kernel by default only when the fold is one small node
        small = p.num_splits <= 16 and p.num_splits * (Hq // Hkv) * D * 4 <= 16384
        assert p.fused == (small and not p.direct)
    assert p.pv_mode == 1  # bf16 MFMA PV unless the tuning selects fp32
    assert p.double_buffer == 0
    assert p.streaming == 1
    assert p.workspace_bytes == expected_workspace(B, Hq, Hkv, D, p)
    again = gd.gqa_decode_plan(B, Hq, Hkv, D, cap, ps, 0, cu)
    assert again.as_dict() == p.as_dict()


@pytest.mark.parametrize("shape", WORKLOAD_SHAPES)
def test_fixed_plan_invariants(tune, shape):
    tune(partition=1)
    B, Hq, Hkv, D, cap, ps = shape
    p = gd.gqa_decode_plan(B, Hq, Hkv, D, cap, ps, 0, 256)
    assert p.partition == 0
    assert p.num_splits * p.split_tokens >= cap
    assert p.grid == B * Hkv * p.num_splits
    assert p.workspace_bytes == expected_workspace(B, Hq, Hkv, D, p)
    if p.num_splits > 1:
        assert p.split_tokens <= 2048


def test_plan_fills_the_device():
    # one kv head, 131072 keys: one workgroup per CU (one sequence: fixed splits)
    p = gd.gqa_decode_plan(1, 8, 1, 128, 131072, 0, 0, 256)
    assert p.partition == 0 and p.grid == 256
    # a batch gets even shares
    p = gd.gqa_decode_plan(32, 32, 8, 128, 8192, 32, 0, 256)
    assert p.partition == 1 and p.grid == 512
    # the GQA-6 layer (4 kv heads, 4096 keys) cannot give every wave more than one tile
    p = gd.gqa_decode_plan(1, 24, 4, 256, 4096, 0, 0, 256)
    assert p.grid == 256 and p.split_tokens == 4 * p.tile_tokens
    # a short cache: one tile per wave over several workgroups where the device has room, the
    # few small partials folded in the split kernel; direct (one workgroup) when it has none
    # (16-key tiles at head_dim 64 there: twice the workgroups)
    p = gd.gqa_decode_plan(1, 8, 2, 64, 512, 0, 0, 256)
    assert p.partition == 0 and p.tile_tokens == 16 and p.num_splits == 8
    assert p.split_tokens == 4 * p.tile_tokens
    assert p.fused == 1 and p.fold_fanin == 8 and p.counters == 2
    p = gd.gqa_decode_plan(64, 32, 8, 128, 256, 0, 0, 256)
    assert p.partition == 0 and p.direct == 1 and p.workspace_bytes == 0
    # with the tile fixed by the tuning, head_dim 64 keeps its 32-key tile
    with gd.tuning(tile_tokens=32):
        p = gd.gqa_decode_plan(1, 8, 2, 64, 512, 0, 0, 256)
    assert p.tile_tokens == 32 and p.num_splits == 4


def test_small_batches_take_fixed_splits():
    """A batch whose one-16-key-tile-per-wave splits take at most four workgroups per CU runs
    them (fixed splits) instead of even shares; past that, and when the tuning asks for even
    shares, the shares stay."""
    for args, splits in (((2, 16, 4, 128, 1024), 16), ((8, 8, 1, 128, 512), 8), ((4, 32, 8, 128, 1024), 16),
                         ((3, 8, 2, 64, 700), 11), ((4, 24, 4, 256, 2048), 32)):
        p = gd.gqa_decode_plan(*args, 0, 0, 256)
        assert p.partition == 0 and p.tile_tokens == 16 and p.num_splits == splits, args
        assert p.split_tokens == 64 and p.grid == args[0] * args[2] * splits
        pp = gd.gqa_decode_plan(*args, 32, 0, 256)          # paged: the same rule
        assert pp.partition == 0 and pp.num_splits == splits
        pf = gd.gqa_decode_plan_fp8(*args, 32, 0, 256)      # E4M3 (32-key paged tiles otherwise)
        assert pf.partition == 0 and pf.tile_tokens == 16 and pf.num_splits == splits
        with gd.tuning(partition=2):
            assert gd.gqa_decode_plan(*args, 0, 0, 256).partition == 1
    # a short batch at head_dim 64 (32-key tiles by default): 16-key tiles, still fixed splits
    p = gd.gqa_decode_plan(2, 16, 4, 64, 512, 0, 0, 256)
    assert p.partition == 0 and p.tile_tokens == 16 and p.num_splits == 8
    p = gd.gqa_decode_plan_fp8(8, 8, 1, 128, 512, 32, 0, 256)
    assert p.partition == 0 and p.tile_tokens == 16 and p.num_splits == 8
    for args in ((16, 32, 8, 128, 1024), (16, 16, 4, 128, 4096), (32, 32, 8, 128, 8192)):
        assert gd.gqa_decode_plan(*args, 0, 0, 256).partition == 1, args
    # fewer CUs: the same job no longer fits four per CU
    assert gd.gqa_decode_plan(4, 32, 8, 128, 1024, 0, 0, 64).partition == 1


def test_proportional_split_plan():
    """partition = 3 (proportional splits): the grid is the share count plus one workgroup per
    segment (each segment's split count is rounded up on the device), every workgroup writes one
    partial slot, the combine is the thread-per-column one, and the E4M3 plan needs no more."""
    with gd.tuning(partition=3):
        p = gd.gqa_decode_plan(16, 32, 4, 128, 16384, 0, 0, 256)
        assert p.partition == 2 and p.num_splits == 0 and p.fused == 0
        assert p.grid == 512 + 64 and p.slots == p.grid
        assert p.split_tokens == 16 * ((64 * 1024 + 511) // 512)      # L tiles at full length
        assert p.max_pieces == 1024 // (p.split_tokens // 16)
        pp = gd.gqa_decode_plan(32, 32, 8, 128, 8192, 32, 0, 256)
        assert pp.partition == 2 and pp.grid == 512 + 256
        pf = gd.gqa_decode_plan_fp8(32, 32, 8, 128, 8192, 32, 0, 256)
        assert pf.partition == 2 and pf.workspace_bytes <= pp.workspace_bytes
        # a single sequence asked for proportional splits takes them too
        p1 = gd.gqa_decode_plan(1, 8, 1, 128, 131072, 0, 0, 256)
        assert p1.partition == 2 and p1.grid == 256 + 1
        # small jobs, forced split counts and short caches keep their fixed plans
        assert gd.gqa_decode_plan(2, 16, 4, 128, 256, 0, 0, 256).partition == 0
        assert gd.gqa_decode_plan(16, 32, 4, 128, 16384, 0, 7, 256).partition == 0


def test_forced_splits_are_clamped_to_tiles():
    p = gd.gqa_decode_plan(1, 8, 2, 64, 512, 0, 1000, 256)
    assert p.partition == 0 and p.num_splits == 512 // p.tile_tokens
    p = gd.gqa_decode_plan(1, 8, 2, 64, 512, 0, 1, 256)
    assert p.num_splits == 1 and p.direct == 1 and p.workspace_bytes == 0
    p = gd.gqa_decode_plan(2, 8, 2, 128, 1000, 0, 7, 256)
    assert p.num_splits == 7


def test_paged_tile_never_straddles_a_page():
    for ps in (16, 32, 48, 64, 80, 128):
        for D in (64, 128, 256):
            p = gd.gqa_decode_plan(4, 8, 2, D, ps * 10, ps, 0, 256)
            assert ps % p.tile_tokens == 0


@pytest.mark.parametrize("args,code", [
    ((1, 8, 3, 128, 100, 0, 0, 256), 2),     # Hq % Hkv != 0
    ((1, 8, 2, 96, 100, 0, 0, 256), 3),      # head_dim 96
    ((1, 34, 2, 128, 100, 0, 0, 256), 3),    # G = 17
    ((1, 8, 2, 128, 100, 24, 0, 256), 3),    # page size not a multiple of 16
    ((1, 8, 2, 128, -1, 0, 0, 256), 2),
    ((1, 8, 2, 128, 100, 0, -1, 256), 2),
    ((1, 8, 2, 128, 100, 0, 0, 0), 2),       # no CUs
])
def test_plan_rejects(args, code):
    with pytest.raises(gd.GqaError) as e:
        gd.gqa_decode_plan(*args)
    assert e.value.code == code


# ---- gqa_decode / gqa_paged_decode argument checks (all fail before any HIP call)
A = 0x10000  # an aligned fake device address; never dereferenced


def call_decode(lib, q=A, k=A, v=A, lens=A, B=1, Hq=8, Hkv=2, D=128, S=64, scale=0.1, out=A,
                ws=A, ws_bytes=1 << 30, splits=2):
    return lib.gqa_decode(q, k, v, lens, B, Hq, Hkv, D, S, scale, out, ws, ws_bytes, splits, None)


def call_paged(lib, q=A, k=A, v=A, lens=A, table=A, B=1, Hq=8, Hkv=2, D=128, ps=32, P=10, mp=4,
               scale=0.1, out=A, ws=A, ws_bytes=1 << 30, splits=2):
    return lib.gqa_paged_decode(q, k, v, lens, table, B, Hq, Hkv, D, ps, P, mp, scale, out, ws,
                                ws_bytes, splits, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(lens=None), 1),
    (dict(out=None), 1), (dict(ws=None), 1),
    (dict(Hq=9), 2), (dict(Hkv=0), 2), (dict(B=-1), 2), (dict(S=-1), 2), (dict(splits=-1), 2),
    (dict(scale=float("nan")), 2), (dict(scale=float("inf")), 2), (dict(S=1 << 30), 2),
    (dict(D=16), 3), (dict(D=80), 3), (dict(Hq=64, Hkv=2), 3),
    (dict(q=A + 8), 4), (dict(k=A + 2), 4), (dict(v=A + 4), 4), (dict(out=A + 4), 4),
    (dict(lens=A + 2), 4), (dict(ws=A + 8), 4),
    (dict(ws_bytes=16), 5),
])
def test_decode_rejects(lib, kw, code):
    assert call_decode(lib, **kw) == code


def test_decode_workspace_exact_size_accepted_without_launch(lib):
    need = gd.gqa_decode_plan(1, 8, 2, 128, 64, 0, 2, 256).workspace_bytes
    assert call_decode(lib, ws_bytes=need - 1) == 5
    # B = 0 passes every check and launches nothing, whatever the pointers
    assert call_decode(lib, B=0, ws_bytes=need) == 0
    assert call_decode(lib, B=0, q=None, k=None, v=None, lens=None, out=None, ws=None) == 0
    assert call_paged(lib, B=0, q=None, table=None, ws=None) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(table=None), 1), (dict(q=None), 1),
    (dict(ps=0), 2), (dict(P=0), 2), (dict(mp=0), 2), (dict(Hq=7), 2),
    (dict(ps=24), 3), (dict(D=48), 3),
    (dict(table=A + 2), 4), (dict(k=A + 8), 4),
    (dict(ws_bytes=0), 5),
])
def test_paged_rejects(lib, kw, code):
    assert call_paged(lib, **kw) == code


def test_workspace_bytes_matches_plan_when_forced(lib):
    for shape in WORKLOAD_SHAPES:
        B, Hq, Hkv, D, cap, ps = shape
        for s in (1, 3, 16):
            assert gd.gqa_decode_workspace_bytes(B, Hq, Hkv, D, cap, ps, s) == \
                gd.gqa_decode_plan(B, Hq, Hkv, D, cap, ps, s, 256).workspace_bytes
    with pytest.raises(gd.GqaError):
        gd.gqa_decode_workspace_bytes(1, 8, 3, 128, 100, 0, 2)


@pytest.mark.parametrize("args,code", [
    (dict(B=1, Hq=8, Hkv=3), 2), (dict(D=96), 3), (dict(out=None), 1), (dict(out=A + 4), 4),
    (dict(ws=None), 1), (dict(ws=A + 8), 4), (dict(ws_bytes=8), 5), (dict(ps=20), 3),
    (dict(lens=None), 1), (dict(lens=A + 2), 4),
    (dict(B=0, out=None, ws=None), 0),          # nothing to do
    (dict(splits=1, ws=None, ws_bytes=0), 0),   # a direct plan has nothing to combine
])
def test_combine_rejects(lib, args, code):
    kw = dict(ws=A, ws_bytes=1 << 30, lens=A, B=1, Hq=8, Hkv=2, D=128, cap=64, ps=0, splits=2,
              out=A)
    kw.update(args)
    assert lib.gqa_decode_combine(kw["ws"], kw["ws_bytes"], kw["lens"], kw["B"], kw["Hq"],
                                  kw["Hkv"], kw["D"], kw["cap"], kw["ps"], kw["splits"], kw["out"],
                                  None) == code


# ---- the E4M3 cache entry points: the same checks, plus finite per-tensor scales
def call_decode_fp8(lib, q=A, k=A, v=A, lens=A, B=1, Hq=8, Hkv=2, D=128, S=64, scale=0.1, ks=1.0,
                    vs=1.0, out=A, ws=A, ws_bytes=1 << 30, splits=2):
    return lib.gqa_decode_fp8(q, k, v, lens, B, Hq, Hkv, D, S, scale, ks, vs, out, ws, ws_bytes,
                              splits, None)


def call_paged_fp8(lib, q=A, k=A, v=A, lens=A, table=A, B=1, Hq=8, Hkv=2, D=128, ps=32, P=10, mp=4,
                   scale=0.1, ks=1.0, vs=1.0, out=A, ws=A, ws_bytes=1 << 30, splits=2):
    return lib.gqa_paged_decode_fp8(q, k, v, lens, table, B, Hq, Hkv, D, ps, P, mp, scale, ks, vs,
                                    out, ws, ws_bytes, splits, None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), 1), (dict(v=None), 1), (dict(lens=None), 1), (dict(out=None), 1),
    (dict(ks=float("nan")), 2), (dict(vs=float("inf")), 2), (dict(ks=float("-inf")), 2),
    (dict(scale=float("nan")), 2), (dict(S=1 << 30), 2), (dict(Hq=9), 2),
    (dict(D=96), 3), (dict(D=32), 3), (dict(k=A + 8), 4), (dict(v=A + 1), 4), (dict(ws_bytes=16), 5),
    (dict(B=0, q=None, k=None, v=None, lens=None, out=None, ws=None), 0),
])
def test_decode_fp8_rejects(lib, kw, code):
    assert call_decode_fp8(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(table=None), 1), (dict(vs=float("nan")), 2), (dict(ps=0), 2), (dict(ps=24), 3),
    (dict(table=A + 2), 4), (dict(ws_bytes=0), 5), (dict(D=32), 3),
])
def test_paged_decode_fp8_rejects(lib, kw, code):
    assert call_paged_fp8(lib, **kw) == code


# ---- multi-query decode: M query tokens per sequence, M * G <= 16 rows per kv head
def call_decode_mq(lib, q=A, k=A, v=A, lens=A, B=1, M=4, Hq=8, Hkv=2, D=128, S=64, scale=0.1,
                   out=A, ws=A, ws_bytes=1 << 30, splits=2):
    return lib.gqa_decode_mq(q, k, v, lens, B, M, Hq, Hkv, D, S, scale, out, ws, ws_bytes, splits,
                             None)


@pytest.mark.parametrize("kw,code", [
    (dict(M=0), 2), (dict(M=-3), 2), (dict(M=5), 3), (dict(M=17, Hq=2, Hkv=2), 3),
    (dict(B=1 << 17, M=4, Hq=16, Hkv=4, D=256, S=64), 2),   # B*M*Hq*D past 32 bits
    (dict(q=None), 1), (dict(q=A + 8), 4), (dict(ws_bytes=16), 5),
    (dict(B=0, q=None, k=None, v=None, lens=None, out=None, ws=None), 0),
])
def test_decode_mq_rejects(lib, kw, code):
    assert call_decode_mq(lib, **kw) == code


def test_mq_workspace_is_the_plan_of_m_times_hq_rows():
    need = gd.gqa_decode_plan(1, 4 * 8, 2, 128, 64, 0, 2, 256).workspace_bytes
    assert need > 0
    assert call_decode_mq(None or gd.load(), ws_bytes=need - 1) == 5


@pytest.mark.parametrize("shape", [
    (32, 32, 8, 128, 8192, 32), (4, 8, 2, 128, 1024, 32), (1, 8, 1, 128, 131072, 64),
    (3, 16, 4, 128, 640, 64), (2, 16, 2, 128, 4096, 16), (5, 24, 4, 256, 2048, 32),
    (6, 16, 4, 64, 512, 32), (16, 32, 4, 128, 16384, 0)])
@pytest.mark.parametrize("splits", [0, 3])
def test_fp8_plan_tiles_and_workspace_bound(shape, splits):
    """The E4M3 plan takes 32-key tiles for a paged head_dim-128 cache (when the page holds
    them; a small job's one-tile-per-wave splits take 16 there too) and 16 otherwise as bf16
    does; its workspace never exceeds the bf16 plan's, which is what gqa_decode_workspace_bytes
    reports for both."""
    B, Hq, Hkv, D, cap, ps = shape
    p16 = gd.gqa_decode_plan(B, Hq, Hkv, D, cap, ps, splits, 256)
    p8 = gd.gqa_decode_plan_fp8(B, Hq, Hkv, D, cap, ps, splits, 256)
    small = splits == 0 and p16.partition == 0 and p16.split_tokens == 4 * p16.tile_tokens == 64
    if ps > 0 and D == 128 and ps % 32 == 0 and not small:
        assert p8.tile_tokens == 32
    else:
        assert p8.tile_tokens == p16.tile_tokens
        assert p8.as_dict() == p16.as_dict()
    assert p8.workspace_bytes <= p16.workspace_bytes
    if ps > 0:
        assert ps % p8.tile_tokens == 0


# ---- tuning: read from the environment once, at load; replaced only by gqa_decode_set_tuning
def test_default_tuning():
    t = gd.gqa_decode_get_tuning().as_dict()
    assert t == dict(tile_tokens=0, double_buffer=0, pv_mode=1, streaming=1, partition=0, shares=0,
                     split_keys=0, piece_cost=4, halve_long=1, combine=0, combine_cols=0,
                     num_splits=0, fold=0, qk_mode=0)


@pytest.mark.parametrize("field,value", [
    ("tile_tokens", 24), ("tile_tokens", 128), ("double_buffer", 2), ("pv_mode", -1),
    ("partition", 4), ("shares", -1), ("piece_cost", 1025), ("combine_cols", 3), ("fold", 3),
    ("num_splits", -2)])
def test_set_tuning_rejects_out_of_range(field, value):
    before = gd.gqa_decode_get_tuning().as_dict()
    t = gd.gqa_decode_get_tuning()
    setattr(t, field, value)
    with pytest.raises(gd.GqaError) as e:
        gd.gqa_decode_set_tuning(t)
    assert e.value.code == 2
    assert gd.gqa_decode_get_tuning().as_dict() == before   # nothing changed
    assert gd.load().gqa_decode_set_tuning(None) == 1


def test_tuning_changes_plans_and_is_restored(tune):
    base = gd.gqa_decode_plan(1, 24, 4, 256, 4096).as_dict()
    tune(num_splits=16, fold=2)
    p = gd.gqa_decode_plan(1, 24, 4, 256, 4096)
    assert p.num_splits == 16 and p.fused == 1 and p.fold_fanin == 16
    assert gd.gqa_decode_workspace_bytes(1, 24, 4, 256, 4096, 0, 16) == p.workspace_bytes
    with gd.tuning(num_splits=0, fold=1):
        assert gd.gqa_decode_plan(1, 24, 4, 256, 4096).as_dict() == base
    assert gd.gqa_decode_plan(1, 24, 4, 256, 4096).num_splits == 16


def test_environment_after_load_changes_nothing(monkeypatch):
    """The GQA_DECODE_* variables are read when the library is loaded, never per call: setting
    them between a *_partials call and its gqa_decode_combine (or between any two calls) cannot
    change the plan, so the combine always reads the partials where the split kernel wrote them."""
    shapes = [(1, 24, 4, 256, 4096, 0), (32, 32, 8, 128, 8192, 32), (3, 16, 4, 128, 1500, 0)]
    before = [gd.gqa_decode_plan(*sh, 0, 256).as_dict() for sh in shapes]
    ws_before = [gd.gqa_decode_workspace_bytes(*sh, 3) for sh in shapes]  # forced: no device query
    for name, value in [("GQA_DECODE_SPLITS", "7"), ("GQA_DECODE_PARTITION", "fixed"),
                        ("GQA_DECODE_SHARES", "3"), ("GQA_DECODE_TILE", "32"),
                        ("GQA_DECODE_FOLD", "fused"), ("GQA_DECODE_PIECE_COST", "0")]:
        monkeypatch.setenv(name, value)
    assert [gd.gqa_decode_plan(*sh, 0, 256).as_dict() for sh in shapes] == before
    assert [gd.gqa_decode_workspace_bytes(*sh, 3) for sh in shapes] == ws_before


def test_environment_is_read_at_load():
    """A fresh process that loads the library with the variables set starts from them."""
    import subprocess
    import sys
    code = ("import decode_attention_04_amd as gd; t = gd.gqa_decode_get_tuning().as_dict(); "
            "print(t['num_splits'], t['partition'], t['fold'], t['shares'], t['pv_mode'], t['tile_tokens'])")
    env = dict(os.environ, GQA_DECODE_SPLITS="7", GQA_DECODE_PARTITION="even", GQA_DECODE_FOLD="fused",
               GQA_DECODE_SHARES="12", GQA_DECODE_PV="f32", GQA_DECODE_TILE="17")  # 17: invalid, ignored
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, check=True).stdout.split()
    assert out == ["7", "2", "2", "12", "0", "0"]


# ---- the in-kernel fold's plan
@pytest.mark.parametrize("S", [2, 5, 16, 17, 64, 100, 256, 1000])
def test_fused_fixed_tree_plan(tune, S):
    """Fixed splits folded in the split kernel: a tree of fan-in F (all S in one node up to 16,
    else the smallest power of two with F * F >= S, at most 16), one counter per node, the inner
    nodes' partials after the splits'; the workspace grows by exactly those."""
    tune(fold=2)
    B, Hq, Hkv, D, cap = 2, 16, 2, 128, 64 * 1024
    p = gd.gqa_decode_plan(B, Hq, Hkv, D, cap, 0, S, 256)
    assert p.partition == 0 and p.fused == 1
    S = p.num_splits   # whole tiles per split: 1000 requested splits become 820
    F = S if S <= 16 else min(16, next(f for f in (2, 4, 8, 16, 32) if f * f >= S))
    assert p.fold_fanin == F
    nodes = tree_nodes(S, F)
    assert p.counters == B * Hkv * nodes and p.counters * 4 <= gd.COUNTER_BYTES
    assert p.slots == B * Hkv * S + B * Hkv * (nodes - 1)
    assert p.workspace_bytes == expected_workspace(B, Hq, Hkv, D, p)
    with gd.tuning(fold=1):
        q = gd.gqa_decode_plan(B, Hq, Hkv, D, cap, 0, S, 256)
        assert q.fused == 0 and q.slots == B * Hkv * S


def test_fused_plans_stay_within_the_counter_header(tune):
    """More (sequence, kv head) segments, or tree nodes, than the header holds: two launches."""
    tune(fold=2)
    p = gd.gqa_decode_plan(4096, 8, 2, 128, 4096, 0, 0, 256)   # 8192 segments, even shares
    assert p.partition == 1 and p.fused == 0 and p.counters == 0
    p = gd.gqa_decode_plan(300, 8, 2, 128, 4096, 0, 64, 256)   # 600 segments x 9 nodes > 4096
    assert p.partition == 0 and p.fused == 0
    p = gd.gqa_decode_plan(100, 8, 2, 128, 4096, 0, 64, 256)   # 200 x 9 = 1800 counters
    assert p.fused == 1 and p.counters == 1800


def test_binding_sizes_a_passed_workspace_without_the_plan():
    """A workspace the caller passes is handed on with its byte size (the library checks it
    against the plan), without a size query; without one, the plan's size is queried, and no
    workspace is made for a plan that needs none."""
    import torch

    def no_query():
        raise AssertionError("size queried although a workspace was passed")

    ws = torch.zeros(100, dtype=torch.float32)
    got, n = gd._workspace(ws, no_query, torch.device("cpu"), None)
    assert got is ws and n == 400
    asked = []
    got, n = gd._workspace(None, lambda: asked.append(1) or 0, torch.device("cpu"), None)
    assert got is None and n == 0 and asked == [1]
    got, n = gd._workspace(None, lambda: 4096, torch.device("cpu"), None)
    assert got.dtype == torch.uint8 and n == 4096 and bool((got == 0).all())
