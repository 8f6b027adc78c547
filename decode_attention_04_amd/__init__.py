"""MI355X (gfx950) GQA flash-decode attention: Python binding over libgqa_decode.so.

The binding only marshals arguments: torch tensors supply device memory and
the current HIP stream, every step of the computation runs in the HIP
kernels of the shared library, and there is no fallback.  If the library is
not built, importing the binding succeeds but every call raises.

Entry points mirror include/gqa_decode.h:
    gqa_decode(q, k_cache, v_cache, seq_lens, scale, ...)
    gqa_paged_decode(q, k_pool, v_pool, seq_lens, page_table, scale, ...)
    gqa_decode_workspace_bytes(B, Hq, Hkv, head_dim, max_seq_len, page_size, num_splits)
    gqa_decode_plan(B, Hq, Hkv, head_dim, max_seq_len, page_size, num_splits, cu_count)
    gqa_decode_partials / gqa_paged_decode_partials + gqa_decode_combine (the two kernels apart)
    gqa_decode_fp8 / gqa_paged_decode_fp8 (+ _partials, gqa_decode_combine_fp8, gqa_decode_plan_fp8)
    gqa_decode_mq / gqa_paged_decode_mq (M query tokens per sequence)
    gqa_decode_noalloc (gqa_decode with the library's static scratch instead of a workspace)
    gqa_decode_get_tuning / gqa_decode_set_tuning, and `tuning(**fields)` (a context manager)
    gqa_status_string(code)
bf16 tensors may be torch.bfloat16 or int16/uint16 views of the bit patterns.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgqa_decode.so")

GQA_OK = 0
# bytes at the start of every workspace that hold the in-kernel fold's arrival counters: they must
# be zero before a workspace is first used (every call leaves them zero)
COUNTER_BYTES = 16384
STATUS_NAMES = {0: "GQA_OK", 1: "GQA_ERR_NULL", 2: "GQA_ERR_SHAPE", 3: "GQA_ERR_UNSUPPORTED",
                4: "GQA_ERR_ALIGN", 5: "GQA_ERR_WORKSPACE", 6: "GQA_ERR_HIP", 7: "GQA_ERR_TOO_LARGE"}

# every symbol include/gqa_decode.h declares
EXPORTED = ("gqa_decode_plan", "gqa_decode_workspace_bytes", "gqa_decode", "gqa_paged_decode",
            "gqa_decode_partials", "gqa_paged_decode_partials", "gqa_decode_combine",
            "gqa_decode_fp8", "gqa_paged_decode_fp8", "gqa_decode_fp8_partials",
            "gqa_paged_decode_fp8_partials", "gqa_decode_plan_fp8", "gqa_decode_combine_fp8",
            "gqa_decode_mq", "gqa_paged_decode_mq", "gqa_decode_get_tuning", "gqa_decode_set_tuning",
            "gqa_decode_noalloc", "gqa_status_string")


class GqaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS_NAMES.get(code, code)} ({gqa_status_string(code)})")


class Plan(ctypes.Structure):
    _fields_ = [("partition", ctypes.c_int), ("num_splits", ctypes.c_int),
                ("split_tokens", ctypes.c_int), ("tile_tokens", ctypes.c_int),
                ("waves", ctypes.c_int), ("grid", ctypes.c_int), ("direct", ctypes.c_int),
                ("max_pieces", ctypes.c_int), ("slots", ctypes.c_int64),
                ("pv_mode", ctypes.c_int),
                ("double_buffer", ctypes.c_int), ("streaming", ctypes.c_int),
                ("workspace_bytes", ctypes.c_size_t), ("fused", ctypes.c_int),
                ("fold_fanin", ctypes.c_int), ("counters", ctypes.c_int64), ("qk_mode", ctypes.c_int)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class Tuning(ctypes.Structure):
    """gqa_tuning_t: the plan and kernel-variant choices (see include/gqa_decode.h)."""
    _fields_ = [(name, ctypes.c_int) for name in (
        "tile_tokens", "double_buffer", "pv_mode", "streaming", "partition", "shares", "split_keys",
        "piece_cost", "halve_long", "combine", "combine_cols", "num_splits", "fold", "qk_mode")]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run decode_attention_04_amd.build.build()")
    lib = ctypes.CDLL(path)
    vp, ci, cf, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.gqa_decode_plan.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci, ctypes.POINTER(Plan)]
    lib.gqa_decode_plan.restype = ci
    lib.gqa_decode_plan_fp8.argtypes = lib.gqa_decode_plan.argtypes
    lib.gqa_decode_plan_fp8.restype = ci
    lib.gqa_decode_workspace_bytes.argtypes = [ci, ci, ci, ci, ci, ci, ci]
    lib.gqa_decode_workspace_bytes.restype = sz
    lib.gqa_decode.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, vp, vp, sz, ci, vp]
    lib.gqa_decode.restype = ci
    lib.gqa_paged_decode.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, vp, vp,
                                     sz, ci, vp]
    lib.gqa_paged_decode.restype = ci
    lib.gqa_decode_partials.argtypes = lib.gqa_decode.argtypes
    lib.gqa_decode_partials.restype = ci
    lib.gqa_paged_decode_partials.argtypes = lib.gqa_paged_decode.argtypes
    lib.gqa_paged_decode_partials.restype = ci
    lib.gqa_decode_combine.argtypes = [vp, sz, vp, ci, ci, ci, ci, ci, ci, ci, vp, vp]
    lib.gqa_decode_combine.restype = ci
    lib.gqa_decode_combine_fp8.argtypes = lib.gqa_decode_combine.argtypes
    lib.gqa_decode_combine_fp8.restype = ci
    lib.gqa_decode_fp8.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, cf, cf, vp, vp, sz, ci, vp]
    lib.gqa_decode_fp8.restype = ci
    lib.gqa_paged_decode_fp8.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, cf, cf, cf,
                                         vp, vp, sz, ci, vp]
    lib.gqa_paged_decode_fp8.restype = ci
    lib.gqa_decode_fp8_partials.argtypes = lib.gqa_decode_fp8.argtypes
    lib.gqa_decode_fp8_partials.restype = ci
    lib.gqa_paged_decode_fp8_partials.argtypes = lib.gqa_paged_decode_fp8.argtypes
    lib.gqa_paged_decode_fp8_partials.restype = ci
    lib.gqa_decode_mq.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp, vp, sz, ci, vp]
    lib.gqa_decode_mq.restype = ci
    lib.gqa_paged_decode_mq.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ci, cf, vp,
                                        vp, sz, ci, vp]
    lib.gqa_paged_decode_mq.restype = ci
    lib.gqa_decode_noalloc.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, vp, ci, vp]
    lib.gqa_decode_noalloc.restype = ci
    lib.gqa_decode_get_tuning.argtypes = [ctypes.POINTER(Tuning)]
    lib.gqa_decode_get_tuning.restype = None
    lib.gqa_decode_set_tuning.argtypes = [ctypes.POINTER(Tuning)]
    lib.gqa_decode_set_tuning.restype = ci
    lib.gqa_status_string.argtypes = [ci]
    lib.gqa_status_string.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def gqa_status_string(code: int) -> str:
    try:
        return load().gqa_status_string(int(code)).decode()
    except RuntimeError:
        return STATUS_NAMES.get(code, str(code))


def gqa_decode_plan(B, Hq, Hkv, head_dim, max_seq_len, page_size=0, num_splits=0, cu_count=256,
                    _entry="gqa_decode_plan"):
    p = Plan()
    rc = getattr(load(), _entry)(B, Hq, Hkv, head_dim, max_seq_len, page_size, num_splits,
                                 cu_count, ctypes.byref(p))
    if rc != GQA_OK:
        raise GqaError(rc, _entry)
    return p


def gqa_decode_plan_fp8(B, Hq, Hkv, head_dim, max_seq_len, page_size=0, num_splits=0, cu_count=256):
    """The plan of a call over an E4M3 cache (paged head_dim 128 takes 32-key tiles)."""
    return gqa_decode_plan(B, Hq, Hkv, head_dim, max_seq_len, page_size, num_splits, cu_count,
                           _entry="gqa_decode_plan_fp8")


def gqa_decode_get_tuning() -> Tuning:
    t = Tuning()
    load().gqa_decode_get_tuning(ctypes.byref(t))
    return t


def gqa_decode_set_tuning(t: Tuning) -> None:
    rc = load().gqa_decode_set_tuning(ctypes.byref(t))
    if rc != GQA_OK:
        raise GqaError(rc, "gqa_decode_set_tuning")


class tuning:
    """Context manager: run the body under the current tuning with some fields replaced, e.g.
    `with tuning(fold=2, shares=7): ...`; the previous tuning is restored on exit."""

    def __init__(self, **fields):
        self.fields = fields

    def __enter__(self):
        self.saved = gqa_decode_get_tuning()
        t = gqa_decode_get_tuning()
        for k, v in self.fields.items():
            if k not in t.as_dict():
                raise KeyError(f"no tuning field {k!r}")
            setattr(t, k, int(v))
        gqa_decode_set_tuning(t)
        return t

    def __exit__(self, *exc):
        gqa_decode_set_tuning(self.saved)
        return False


def gqa_decode_workspace_bytes(B, Hq, Hkv, head_dim, max_seq_len, page_size=0, num_splits=0):
    n = load().gqa_decode_workspace_bytes(B, Hq, Hkv, head_dim, max_seq_len, page_size,
                                          num_splits)
    if n == ctypes.c_size_t(-1).value:
        raise GqaError(2, "gqa_decode_workspace_bytes")
    return n


# ------------------------------------------------------------------ tensor marshalling
# Per-call marshalling is on the host's critical path for eager callers (a call of the
# binding costs more host time than the two kernel launches it makes), so the torch
# module, the dtype sets and the raw current-stream query are looked up once.
_TORCH = None
_BF16_TYPES = None
_RAW_STREAM = None  # torch's raw current-stream query, when this torch build has it


def _torch():
    global _TORCH, _BF16_TYPES, _RAW_STREAM
    if _TORCH is None:
        import torch
        _BF16_TYPES = (torch.bfloat16, torch.int16, torch.uint16)
        _RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _TORCH = torch
    return _TORCH


def _dev_ptr(t, name, dtypes):
    if not isinstance(t, _torch().Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _bf16_types():
    _torch()
    return _BF16_TYPES


def _stream_ptr(stream, device):
    """The raw hipStream_t of `stream`, else of the current stream of `device` (a tensor's
    device)."""
    if stream is not None:
        return stream.cuda_stream
    torch = _torch()
    if _RAW_STREAM is not None and device.type == "cuda" and device.index is not None:
        return _RAW_STREAM(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _alloc(shape, dtype, device, stream, zero=False):
    """A buffer the binding allocates for one call.  It is allocated on the stream the kernels
    run on: the caching allocator then never hands its memory to other work until that stream
    has passed the kernels, even after the tensor is dropped."""
    torch = _torch()
    make = torch.zeros if zero else torch.empty
    if stream is None:
        return make(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return make(shape, dtype=dtype, device=device)


def new_workspace(nbytes, device="cuda", stream=None):
    """A workspace for gqa_* calls: zero-filled (its arrival counters must start at zero; every
    call leaves them zero again), reusable by any later call of any shape on the same stream."""
    return _alloc(max(int(nbytes), 0), _torch().uint8, device, stream, zero=True)


def _workspace(workspace, need, device, stream):
    """(workspace, its bytes): the caller's, whose size the library checks against the plan,
    or one allocated for the call when `need()` (the plan's bytes) is not 0."""
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    n = need()
    if n == 0:
        return None, 0
    workspace = new_workspace(n, device, stream)
    return workspace, workspace.numel() * workspace.element_size()


def gqa_decode(q, k_cache, v_cache, seq_lens, scale, out=None, workspace=None, num_splits=0,
               stream=None, _entry="gqa_decode"):
    """Contiguous cache: q [B,Hq,D], k/v [B,Hkv,S_max,D] bf16, seq_lens int32 [B].

    Returns out (fp32 [B,Hq,D]).  `workspace` (a uint8 device tensor from new_workspace, or any
    buffer whose first 16384 bytes are zero) is allocated when not given; pass one to keep the
    call allocation-free."""
    torch = _torch()
    B, Hq, D = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    if out is None:
        out = _alloc((B, Hq, D), torch.float32, q.device, stream)
    need = lambda: gqa_decode_workspace_bytes(B, Hq, Hkv, D, S_max, 0, num_splits)
    workspace, ws_bytes = _workspace(workspace, need, q.device, stream)
    bf = _bf16_types()
    rc = getattr(load(), _entry)(
        _dev_ptr(q, "q", bf), _dev_ptr(k_cache, "k_cache", bf), _dev_ptr(v_cache, "v_cache", bf),
        _dev_ptr(seq_lens, "seq_lens", (torch.int32,)), B, Hq, Hkv, D, S_max, float(scale),
        _dev_ptr(out, "out", (torch.float32,)),
        None if workspace is None else workspace.data_ptr(), ws_bytes, int(num_splits),
        _stream_ptr(stream, q.device))
    if rc != GQA_OK:
        raise GqaError(rc, _entry)
    return out


def gqa_paged_decode(q, k_pool, v_pool, seq_lens, page_table, scale, out=None, workspace=None,
                     num_splits=0, stream=None, _entry="gqa_paged_decode"):
    """Paged cache: k/v pools [P,Hkv,page_size,D] bf16, page_table int32 [B,max_pages]."""
    torch = _torch()
    B, Hq, D = q.shape
    P, Hkv, page_size, _ = k_pool.shape
    max_pages = page_table.shape[1]
    if out is None:
        out = _alloc((B, Hq, D), torch.float32, q.device, stream)
    need = lambda: gqa_decode_workspace_bytes(B, Hq, Hkv, D, max_pages * page_size, page_size, num_splits)
    workspace, ws_bytes = _workspace(workspace, need, q.device, stream)
    bf = _bf16_types()
    rc = getattr(load(), _entry)(
        _dev_ptr(q, "q", bf), _dev_ptr(k_pool, "k_pool", bf), _dev_ptr(v_pool, "v_pool", bf),
        _dev_ptr(seq_lens, "seq_lens", (torch.int32,)),
        _dev_ptr(page_table, "page_table", (torch.int32,)), B, Hq, Hkv, D, page_size, P,
        max_pages, float(scale), _dev_ptr(out, "out", (torch.float32,)),
        None if workspace is None else workspace.data_ptr(), ws_bytes, int(num_splits),
        _stream_ptr(stream, q.device))
    if rc != GQA_OK:
        raise GqaError(rc, _entry)
    return out


def _fp8_types():
    torch = _torch()
    return tuple(t for t in (torch.uint8, getattr(torch, "float8_e4m3fn", None)) if t is not None)


def gqa_decode_fp8(q, k_cache, v_cache, seq_lens, scale, k_scale, v_scale, out=None,
                   workspace=None, num_splits=0, stream=None, _entry="gqa_decode_fp8"):
    """Contiguous E4M3 cache: k/v [B,Hkv,S_max,D] uint8 (or float8_e4m3fn) bytes, one fp32
    scale per tensor; otherwise as gqa_decode."""
    torch = _torch()
    B, Hq, D = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    if out is None:
        out = _alloc((B, Hq, D), torch.float32, q.device, stream)
    need = lambda: gqa_decode_workspace_bytes(B, Hq, Hkv, D, S_max, 0, num_splits)
    workspace, ws_bytes = _workspace(workspace, need, q.device, stream)
    f8 = _fp8_types()
    rc = getattr(load(), _entry)(
        _dev_ptr(q, "q", _bf16_types()), _dev_ptr(k_cache, "k_cache", f8),
        _dev_ptr(v_cache, "v_cache", f8), _dev_ptr(seq_lens, "seq_lens", (torch.int32,)), B, Hq,
        Hkv, D, S_max, float(scale), float(k_scale), float(v_scale),
        _dev_ptr(out, "out", (torch.float32,)),
        None if workspace is None else workspace.data_ptr(), ws_bytes, int(num_splits),
        _stream_ptr(stream, q.device))
    if rc != GQA_OK:
        raise GqaError(rc, _entry)
    return out


def gqa_paged_decode_fp8(q, k_pool, v_pool, seq_lens, page_table, scale, k_scale, v_scale,
                         out=None, workspace=None, num_splits=0, stream=None,
                         _entry="gqa_paged_decode_fp8"):
    """Paged E4M3 cache: k/v pools [P,Hkv,page_size,D] uint8 (or float8_e4m3fn) bytes."""
    torch = _torch()
    B, Hq, D = q.shape
    P, Hkv, page_size, _ = k_pool.shape
    max_pages = page_table.shape[1]
    if out is None:
        out = _alloc((B, Hq, D), torch.float32, q.device, stream)
    need = lambda: gqa_decode_workspace_bytes(B, Hq, Hkv, D, max_pages * page_size, page_size, num_splits)
    workspace, ws_bytes = _workspace(workspace, need, q.device, stream)
    f8 = _fp8_types()
    rc = getattr(load(), _entry)(
        _dev_ptr(q, "q", _bf16_types()), _dev_ptr(k_pool, "k_pool", f8),
        _dev_ptr(v_pool, "v_pool", f8), _dev_ptr(seq_lens, "seq_lens", (torch.int32,)),
        _dev_ptr(page_table, "page_table", (torch.int32,)), B, Hq, Hkv, D, page_size, P,
        max_pages, float(scale), float(k_scale), float(v_scale),
        _dev_ptr(out, "out", (torch.float32,)),
        None if workspace is None else workspace.data_ptr(), ws_bytes, int(num_splits),
        _stream_ptr(stream, q.device))
    if rc != GQA_OK:
        raise GqaError(rc, _entry)
    return out


def gqa_decode_fp8_partials(q, k_cache, v_cache, seq_lens, scale, k_scale, v_scale, out=None,
                            workspace=None, num_splits=0, stream=None):
    """The split kernel of gqa_decode_fp8 alone (partials into `workspace`, which must be given)."""
    if workspace is None:
        raise ValueError("gqa_decode_fp8_partials needs the workspace the combine will read")
    return gqa_decode_fp8(q, k_cache, v_cache, seq_lens, scale, k_scale, v_scale, out, workspace,
                          num_splits, stream, _entry="gqa_decode_fp8_partials")


def gqa_paged_decode_fp8_partials(q, k_pool, v_pool, seq_lens, page_table, scale, k_scale,
                                  v_scale, out=None, workspace=None, num_splits=0, stream=None):
    """The split kernel of gqa_paged_decode_fp8 alone."""
    if workspace is None:
        raise ValueError("gqa_paged_decode_fp8_partials needs the workspace the combine will read")
    return gqa_paged_decode_fp8(q, k_pool, v_pool, seq_lens, page_table, scale, k_scale, v_scale,
                                out, workspace, num_splits, stream,
                                _entry="gqa_paged_decode_fp8_partials")


def gqa_decode_mq(q, k_cache, v_cache, seq_lens, scale, out=None, workspace=None, num_splits=0,
                  stream=None):
    """Multi-query decode: q [B,M,Hq,D] bf16 (the last M positions of each sequence, query i
    attending to keys 0 .. len-M+i), k/v [B,Hkv,S_max,D]; returns out fp32 [B,M,Hq,D]."""
    torch = _torch()
    B, M, Hq, D = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    if out is None:
        out = _alloc((B, M, Hq, D), torch.float32, q.device, stream)
    need = lambda: gqa_decode_workspace_bytes(B, M * Hq, Hkv, D, S_max, 0, num_splits)
    workspace, ws_bytes = _workspace(workspace, need, q.device, stream)
    bf = _bf16_types()
    rc = load().gqa_decode_mq(
        _dev_ptr(q, "q", bf), _dev_ptr(k_cache, "k_cache", bf), _dev_ptr(v_cache, "v_cache", bf),
        _dev_ptr(seq_lens, "seq_lens", (torch.int32,)), B, M, Hq, Hkv, D, S_max, float(scale),
        _dev_ptr(out, "out", (torch.float32,)),
        None if workspace is None else workspace.data_ptr(), ws_bytes, int(num_splits),
        _stream_ptr(stream, q.device))
    if rc != GQA_OK:
        raise GqaError(rc, "gqa_decode_mq")
    return out


def gqa_paged_decode_mq(q, k_pool, v_pool, seq_lens, page_table, scale, out=None, workspace=None,
                        num_splits=0, stream=None):
    """Multi-query decode over a paged cache: q [B,M,Hq,D]."""
    torch = _torch()
    B, M, Hq, D = q.shape
    P, Hkv, page_size, _ = k_pool.shape
    max_pages = page_table.shape[1]
    if out is None:
        out = _alloc((B, M, Hq, D), torch.float32, q.device, stream)
    need = lambda: gqa_decode_workspace_bytes(B, M * Hq, Hkv, D, max_pages * page_size, page_size,
                                      num_splits)
    workspace, ws_bytes = _workspace(workspace, need, q.device, stream)
    bf = _bf16_types()
    rc = load().gqa_paged_decode_mq(
        _dev_ptr(q, "q", bf), _dev_ptr(k_pool, "k_pool", bf), _dev_ptr(v_pool, "v_pool", bf),
        _dev_ptr(seq_lens, "seq_lens", (torch.int32,)),
        _dev_ptr(page_table, "page_table", (torch.int32,)), B, M, Hq, Hkv, D, page_size, P,
        max_pages, float(scale), _dev_ptr(out, "out", (torch.float32,)),
        None if workspace is None else workspace.data_ptr(), ws_bytes, int(num_splits),
        _stream_ptr(stream, q.device))
    if rc != GQA_OK:
        raise GqaError(rc, "gqa_paged_decode_mq")
    return out


def gqa_decode_partials(q, k_cache, v_cache, seq_lens, scale, out=None, workspace=None,
                        num_splits=0, stream=None):
    """The split kernel of gqa_decode alone (partials into `workspace`, which must be given)."""
    if workspace is None:
        raise ValueError("gqa_decode_partials needs the workspace the combine will read")
    return gqa_decode(q, k_cache, v_cache, seq_lens, scale, out, workspace, num_splits, stream,
                      _entry="gqa_decode_partials")


def gqa_paged_decode_partials(q, k_pool, v_pool, seq_lens, page_table, scale, out=None,
                              workspace=None, num_splits=0, stream=None):
    """The split kernel of gqa_paged_decode alone (partials into `workspace`)."""
    if workspace is None:
        raise ValueError("gqa_paged_decode_partials needs the workspace the combine will read")
    return gqa_paged_decode(q, k_pool, v_pool, seq_lens, page_table, scale, out, workspace,
                            num_splits, stream, _entry="gqa_paged_decode_partials")


def gqa_decode_combine(workspace, seq_lens, out, B, Hq, Hkv, head_dim, max_seq_len, page_size=0,
                       num_splits=0, stream=None, _entry="gqa_decode_combine"):
    """Fold the partials a *_partials call left in `workspace` into `out`."""
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = getattr(load(), _entry)(ws_ptr, ws_bytes,
                                 _dev_ptr(seq_lens, "seq_lens", (_torch().int32,)), B, Hq, Hkv,
                                 head_dim, max_seq_len, page_size, num_splits,
                                 _dev_ptr(out, "out", (_torch().float32,)),
                                 _stream_ptr(stream, out.device))
    if rc != GQA_OK:
        raise GqaError(rc, _entry)
    return out


def gqa_decode_combine_fp8(workspace, seq_lens, out, B, Hq, Hkv, head_dim, max_seq_len, page_size=0,
                           num_splits=0, stream=None):
    """Fold the partials a gqa_*_fp8_partials call left in `workspace` into `out`."""
    return gqa_decode_combine(workspace, seq_lens, out, B, Hq, Hkv, head_dim, max_seq_len,
                              page_size, num_splits, stream, _entry="gqa_decode_combine_fp8")


def gqa_decode_noalloc(q, k_cache, v_cache, seq_lens, scale, out, num_splits=0, stream=None):
    """gqa_decode without a workspace: the partials live in the library's static per-GPU scratch
    (4 MiB), so the call allocates nothing; `out` (fp32 [B,Hq,D]) must be given."""
    torch = _torch()
    B, Hq, D = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    bf = _bf16_types()
    rc = load().gqa_decode_noalloc(
        _dev_ptr(q, "q", bf), _dev_ptr(k_cache, "k_cache", bf), _dev_ptr(v_cache, "v_cache", bf),
        _dev_ptr(seq_lens, "seq_lens", (torch.int32,)), B, Hq, Hkv, D, S_max, float(scale),
        _dev_ptr(out, "out", (torch.float32,)), int(num_splits), _stream_ptr(stream, q.device))
    if rc != GQA_OK:
        raise GqaError(rc, "gqa_decode_noalloc")
    return out
