"""Helpers for the GPU parity tests: upload a Case, call the C ABI, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import decode_attention_04_amd as gd
from tests import workloads as W

ATOL = 2e-3
RTOL = 2e-3


def require_gpu():
    assert torch.cuda.is_available(), "this test needs an MI355X GPU"
    gd.load()  # raises if the HIP library is not built


def dev_bf16(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


def dev_u8(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


def dev_i32(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


class DeviceCase:
    """A Case resident in device memory."""

    def __init__(self, case: W.Case, device="cuda"):
        self.case = case
        self.q = dev_bf16(case.q, device)
        cache = dev_u8 if case.kv == "fp8" else dev_bf16
        self.k = cache(case.k, device)
        self.v = cache(case.v, device)
        self.seq_lens = dev_i32(case.seq_lens, device)
        self.page_table = dev_i32(case.page_table, device) if case.paged else None

    def run(self, num_splits=0, out=None, workspace=None, stream=None) -> torch.Tensor:
        c = self.case
        if c.M > 1:
            if c.paged:
                return gd.gqa_paged_decode_mq(self.q, self.k, self.v, self.seq_lens, self.page_table,
                                              c.scale, out=out, workspace=workspace,
                                              num_splits=num_splits, stream=stream)
            return gd.gqa_decode_mq(self.q, self.k, self.v, self.seq_lens, c.scale, out=out,
                                    workspace=workspace, num_splits=num_splits, stream=stream)
        if c.kv == "fp8":
            if c.paged:
                return gd.gqa_paged_decode_fp8(self.q, self.k, self.v, self.seq_lens,
                                               self.page_table, c.scale, c.k_scale, c.v_scale,
                                               out=out, workspace=workspace,
                                               num_splits=num_splits, stream=stream)
            return gd.gqa_decode_fp8(self.q, self.k, self.v, self.seq_lens, c.scale, c.k_scale,
                                     c.v_scale, out=out, workspace=workspace,
                                     num_splits=num_splits, stream=stream)
        if c.paged:
            return gd.gqa_paged_decode(self.q, self.k, self.v, self.seq_lens, self.page_table,
                                       c.scale, out=out, workspace=workspace,
                                       num_splits=num_splits, stream=stream)
        return gd.gqa_decode(self.q, self.k, self.v, self.seq_lens, c.scale, out=out,
                             workspace=workspace, num_splits=num_splits, stream=stream)

    def run_host(self, num_splits=0) -> np.ndarray:
        out = self.run(num_splits)
        torch.cuda.synchronize()
        return out.cpu().numpy()


def oracle_out(case: W.Case) -> np.ndarray:
    import oracle
    if case.M > 1:
        if case.paged:
            return oracle.paged_decode_mq(case.q, case.k, case.v, case.seq_lens, case.page_table,
                                          case.scale)
        return oracle.decode_mq(case.q, case.k, case.v, case.seq_lens, case.scale)
    if case.kv == "fp8":
        if case.paged:
            return oracle.paged_decode_fp8(case.q, case.k, case.v, case.seq_lens, case.page_table,
                                           case.scale, case.k_scale, case.v_scale)
        return oracle.decode_fp8(case.q, case.k, case.v, case.seq_lens, case.scale, case.k_scale,
                                 case.v_scale)
    if case.paged:
        return oracle.paged_decode(case.q, case.k, case.v, case.seq_lens, case.page_table,
                                   case.scale)
    return oracle.decode(case.q, case.k, case.v, case.seq_lens, case.scale)


def compare(gpu: np.ndarray, ref: np.ndarray, what: str = "", atol=ATOL, rtol=RTOL) -> dict:
    """Elementwise |gpu - ref| <= atol + rtol |ref|; returns error statistics."""
    gpu = np.asarray(gpu, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    err = np.abs(gpu - ref)
    bad = err > atol + rtol * np.abs(ref)
    big = np.abs(ref) >= 1e-3
    stats = {"max_abs": float(err.max(initial=0)),
             "max_rel": float((err[big] / np.abs(ref[big])).max(initial=0)),
             "n_bad": int(bad.sum()), "n": int(err.size)}
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), err.shape)
        raise AssertionError(f"{what}: {stats['n_bad']}/{err.size} outside tolerance; worst at "
                             f"{i}: gpu={gpu[i]!r} oracle={ref[i]!r}; {stats}")
    return stats
