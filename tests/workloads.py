"""Seeded synthetic inputs for GQA flash-decode (shared by the tests and bench.py).

This module holds no attention arithmetic: it only draws random numbers,
rounds them to bf16 bit patterns, and lays them out as the caches the
library reads.  Both the oracle and the HIP path consume exactly these bytes.

Recipe (all five named workloads):
  * numpy.random.default_rng(seed) (seed 0 unless stated), draws in the order
    q, K, V, then sequence lengths, then the page permutation, then the
    indices of the amplified keys;
  * q, K, V ~ N(0, 1) drawn as float32 and rounded to bf16 (round to nearest
    even), scale = float32(1 / sqrt(head_dim));
  * contiguous caches are [B][Hkv][S_max][D] with S_max = the context length;
  * the paged workload draws lengths uniformly from the integers 1..8192, and
    hands sequence 0 the first ceil(len0/32) entries of one random
    permutation of the 10000 pool pages, sequence 1 the next, and so on;
    unused table entries are -1;
  * the peaky long-context workload multiplies the whole key row of
    floor(1% of the context) distinct token positions by 8 (exact in bf16).

FP8 caches (the quantized-KV variant): q as above; K and V ~ N(0, 1) drawn
as float32, divided by their per-tensor scale (1/16 unless stated, a power of
two) and rounded to the nearest OCP FP8 E4M3 value (ties to an even
mantissa, saturating at +-448), stored as uint8 bytes.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even; NaN -> quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    out = np.empty(x.shape, np.uint16)
    step = 1 << 22
    for i in range(0, x.size, step):
        u = x[i:i + step].view(np.uint32).copy()
        t = u >> np.uint32(16)
        t &= np.uint32(1)
        t += np.uint32(0x7FFF)
        u += t
        u >>= np.uint32(16)
        out[i:i + step] = u
        nan = np.isnan(x[i:i + step])
        if nan.any():
            out[i:i + step][nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- fp8 (E4M3) bytes
def _e4m3_grid() -> np.ndarray:
    """Values of the bytes 0x00 .. 0x7E (all finite non-negative E4M3 values, ascending)."""
    b = np.arange(127)
    e, m = (b >> 3) & 0xF, b & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7)).astype(np.float64)


_E4M3 = _e4m3_grid()


def f32_to_e4m3_bytes(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP FP8 E4M3 bytes: nearest value, ties to an even mantissa, saturating
    at +-448; NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64).reshape(-1)
    hi = np.clip(np.searchsorted(_E4M3, a), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    dlo, dhi = np.abs(a - _E4M3[lo]), np.abs(_E4M3[hi] - a)
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a >= _E4M3[126], 126, pick).astype(np.uint8)
    out = pick | np.where(np.signbit(x.reshape(-1)), 0x80, 0).astype(np.uint8)
    out[np.isnan(x.reshape(-1))] = 0x7F
    return out.reshape(x.shape)


def _normal_fp8(rng: np.random.Generator, shape, kv_scale: float) -> np.ndarray:
    out = np.empty(shape, np.uint8)
    flat = out.reshape(-1)
    n, step = flat.size, 1 << 22
    for i in range(0, n, step):
        m = min(step, n - i)
        flat[i:i + m] = f32_to_e4m3_bytes(rng.standard_normal(m, dtype=np.float32) / np.float32(kv_scale))
    return out


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32)).reshape(shape)


# ---------------------------------------------------------------- cases
@dataclasses.dataclass
class Case:
    """One decode call's inputs. bf16 tensors are uint16 bit patterns."""
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    scale: float                  # a float32 value
    q: np.ndarray                 # [B, Hq, D]
    k: np.ndarray                 # contiguous [B, Hkv, S_max, D] or pool [P, Hkv, ps, D]
    v: np.ndarray
    seq_lens: np.ndarray          # int32 [B]
    page_table: np.ndarray | None = None   # int32 [B, max_pages] (paged only)
    page_size: int = 0
    kv: str = "bf16"              # "bf16": k, v are uint16 bf16 bits; "fp8": uint8 E4M3 bytes
    k_scale: float = 1.0          # fp8: per-tensor scales (float32 values)
    v_scale: float = 1.0
    M: int = 1                    # query tokens per sequence; M > 1: q is [B, M, Hq, D]

    @property
    def paged(self) -> bool:
        return self.page_table is not None

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def S_max(self) -> int:
        return 0 if self.paged else self.k.shape[2]

    @property
    def num_pages(self) -> int:
        return self.k.shape[0] if self.paged else 0

    @property
    def max_pages(self) -> int:
        return self.page_table.shape[1] if self.paged else 0

    @property
    def capacity(self) -> int:
        """Largest sequence length the cache can hold."""
        return self.max_pages * self.page_size if self.paged else self.S_max

    @property
    def kv_bytes(self) -> int:
        """Bytes per cache element (2 for bf16, 1 for fp8)."""
        return 1 if self.kv == "fp8" else 2

    def algorithmic_bytes(self) -> int:
        """sum(len) * Hkv * D * 2 (K and V) * element bytes + q (bf16) + out (fp32)."""
        return (int(self.seq_lens.astype(np.int64).sum()) * self.Hkv * self.D * 2 * self.kv_bytes
                + self.B * self.M * self.Hq * self.D * (2 + 4))


def default_scale(D: int) -> float:
    return float(np.float32(1.0 / math.sqrt(D)))


def contig_case(B, Hq, Hkv, D, S_max, seq_lens=None, *, seed=0, scale=None, tail=None,
                name="contig") -> Case:
    """Contiguous cache.  seq_lens defaults to S_max for every sequence.
    tail: None leaves rows >= len as drawn; "nan" poisons them with NaN;
    "inf" with +inf."""
    return _contig(np.random.default_rng(seed), B, Hq, Hkv, D, S_max, seq_lens, scale, tail, name)


def _contig(rng, B, Hq, Hkv, D, S_max, seq_lens, scale, tail, name) -> Case:
    q = _normal_bf16(rng, (B, Hq, D))
    k = _normal_bf16(rng, (B, Hkv, S_max, D))
    v = _normal_bf16(rng, (B, Hkv, S_max, D))
    lens = np.full(B, S_max, np.int32) if seq_lens is None else np.asarray(seq_lens, np.int32)
    if tail is not None:
        fill = {"nan": 0x7FC0, "inf": 0x7F80}[tail]
        for b in range(B):
            k[b, :, lens[b]:, :] = fill
            v[b, :, lens[b]:, :] = fill
    return Case(name, B, Hq, Hkv, D, default_scale(D) if scale is None else float(np.float32(scale)),
                q, k, v, lens)


def fp8_contig_case(B, Hq, Hkv, D, S_max, seq_lens=None, *, seed=0, scale=None, k_scale=1 / 16,
                    v_scale=1 / 16, tail=None, name="fp8_contig") -> Case:
    """Contiguous E4M3 cache with per-tensor scales.  tail "nan" poisons rows >= len (0x7F)."""
    rng = np.random.default_rng(seed)
    q = _normal_bf16(rng, (B, Hq, D))
    k = _normal_fp8(rng, (B, Hkv, S_max, D), k_scale)
    v = _normal_fp8(rng, (B, Hkv, S_max, D), v_scale)
    lens = np.full(B, S_max, np.int32) if seq_lens is None else np.asarray(seq_lens, np.int32)
    if tail == "nan":
        for b in range(B):
            k[b, :, lens[b]:, :] = 0x7F
            v[b, :, lens[b]:, :] = 0x7F
    return Case(name, B, Hq, Hkv, D, default_scale(D) if scale is None else float(np.float32(scale)),
                q, k, v, lens, kv="fp8", k_scale=float(np.float32(k_scale)),
                v_scale=float(np.float32(v_scale)))


def fp8_paged_case(B, Hq, Hkv, D, page_size, num_pages, seq_lens=None, *, max_len=None, seed=0,
                   scale=None, k_scale=1 / 16, v_scale=1 / 16, max_pages=None,
                   name="fp8_paged") -> Case:
    """Paged E4M3 cache.  If seq_lens is None they are drawn uniformly from 1..max_len."""
    rng = np.random.default_rng(seed)
    q = _normal_bf16(rng, (B, Hq, D))
    k = _normal_fp8(rng, (num_pages, Hkv, page_size, D), k_scale)
    v = _normal_fp8(rng, (num_pages, Hkv, page_size, D), v_scale)
    if seq_lens is None:
        lens = rng.integers(1, max_len, size=B, endpoint=True).astype(np.int32)
    else:
        lens = np.asarray(seq_lens, np.int32)
    cap = max_len if max_len is not None else int(lens.max(initial=0))
    if max_pages is None:
        max_pages = max(1, (cap + page_size - 1) // page_size)
    table = assign_pages(rng, lens, page_size, num_pages, max_pages)
    return Case(name, B, Hq, Hkv, D, default_scale(D) if scale is None else float(np.float32(scale)),
                q, k, v, lens, table, page_size, kv="fp8", k_scale=float(np.float32(k_scale)),
                v_scale=float(np.float32(v_scale)))


def mq_case(B, M, Hq, Hkv, D, S_max, seq_lens=None, *, seed=0, scale=None, tail=None,
            name="mq") -> Case:
    """Multi-query decode over a contiguous cache: q [B, M, Hq, D], the last M positions of each
    sequence.  tail "nan" poisons rows >= len."""
    rng = np.random.default_rng(seed)
    q = _normal_bf16(rng, (B, M, Hq, D))
    k = _normal_bf16(rng, (B, Hkv, S_max, D))
    v = _normal_bf16(rng, (B, Hkv, S_max, D))
    lens = np.full(B, S_max, np.int32) if seq_lens is None else np.asarray(seq_lens, np.int32)
    if tail == "nan":
        for b in range(B):
            k[b, :, lens[b]:, :] = 0x7FC0
            v[b, :, lens[b]:, :] = 0x7FC0
    return Case(name, B, Hq, Hkv, D, default_scale(D) if scale is None else float(np.float32(scale)),
                q, k, v, lens, M=M)


def mq_paged_case(B, M, Hq, Hkv, D, page_size, num_pages, seq_lens, *, max_len, seed=0,
                  scale=None, name="mq_paged") -> Case:
    """Multi-query decode over a paged cache."""
    rng = np.random.default_rng(seed)
    q = _normal_bf16(rng, (B, M, Hq, D))
    k = _normal_bf16(rng, (num_pages, Hkv, page_size, D))
    v = _normal_bf16(rng, (num_pages, Hkv, page_size, D))
    lens = np.asarray(seq_lens, np.int32)
    table = assign_pages(rng, lens, page_size, num_pages, max(1, (max_len + page_size - 1) // page_size))
    return Case(name, B, Hq, Hkv, D, default_scale(D) if scale is None else float(np.float32(scale)),
                q, k, v, lens, table, page_size, M=M)


def assign_pages(rng: np.random.Generator, lens, page_size: int, num_pages: int,
                 max_pages: int) -> np.ndarray:
    """Consecutive slices of one random permutation of the pool, -1 elsewhere."""
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.full((len(lens), max_pages), -1, np.int32)
    pos = 0
    for b, n in enumerate(lens):
        used = (int(n) + page_size - 1) // page_size
        if used > max_pages or pos + used > num_pages:
            raise ValueError("pool too small for the requested lengths")
        table[b, :used] = perm[pos:pos + used]
        pos += used
    return table


def paged_case(B, Hq, Hkv, D, page_size, num_pages, seq_lens=None, *, max_len=None, seed=0,
               scale=None, max_pages=None, name="paged") -> Case:
    """Paged cache.  If seq_lens is None they are drawn uniformly from 1..max_len."""
    rng = np.random.default_rng(seed)
    q = _normal_bf16(rng, (B, Hq, D))
    k = _normal_bf16(rng, (num_pages, Hkv, page_size, D))
    v = _normal_bf16(rng, (num_pages, Hkv, page_size, D))
    if seq_lens is None:
        lens = rng.integers(1, max_len, size=B, endpoint=True).astype(np.int32)
    else:
        lens = np.asarray(seq_lens, np.int32)
    cap = max_len if max_len is not None else int(lens.max(initial=0))
    if max_pages is None:
        max_pages = max(1, (cap + page_size - 1) // page_size)
    table = assign_pages(rng, lens, page_size, num_pages, max_pages)
    return Case(name, B, Hq, Hkv, D, default_scale(D) if scale is None else float(np.float32(scale)),
                q, k, v, lens, table, page_size)


def peaky_case(B, Hq, Hkv, D, S_max, *, frac=0.01, mul=8, seed=0, name="peaky") -> Case:
    """Contiguous cache whose key rows at floor(frac*S_max) random positions are scaled by mul."""
    rng = np.random.default_rng(seed)
    c = _contig(rng, B, Hq, Hkv, D, S_max, None, None, None, name)
    idx = rng.choice(S_max, size=int(math.floor(frac * S_max)), replace=False)
    kf = bf16_bits_to_f32(c.k[:, :, idx, :]) * np.float32(mul)
    c.k[:, :, idx, :] = f32_to_bf16_bits(kf).reshape(kf.shape)
    return c


# ---------------------------------------------------------------- the five workloads
WORKLOADS = {
    # tiny contiguous GQA decode, G=4, seed 0
    "tiny_gqa4_d64_ctx512": lambda seed=0: contig_case(
        1, 8, 2, 64, 512, seed=seed, name="tiny_gqa4_d64_ctx512"),
    # GQA-6 long-context layer: the kernel the sparkinfer pages profile
    "gqa6_d256_ctx4096": lambda seed=0: contig_case(
        1, 24, 4, 256, 4096, seed=seed, scale=1.0 / 16, name="gqa6_d256_ctx4096"),
    # batched GQA-8
    "batched_gqa8_d128_ctx16k": lambda seed=0: contig_case(
        16, 32, 4, 128, 16384, seed=seed, name="batched_gqa8_d128_ctx16k"),
    # ragged paged batch, G=4, page_size 32, 10000-page pool
    "paged_gqa4_d128_ragged8k": lambda seed=0: paged_case(
        32, 32, 8, 128, 32, 10000, max_len=8192, seed=seed, name="paged_gqa4_d128_ragged8k"),
    # one very long sequence with a peaky softmax
    "long_gqa8_d128_ctx128k_peaky": lambda seed=0: peaky_case(
        1, 8, 1, 128, 131072, seed=seed, name="long_gqa8_d128_ctx128k_peaky"),
}

# the workload the headline benchmark line is quoted on
HEADLINE = "gqa6_d256_ctx4096"


# per-tensor scales of the E4M3 form of each workload: 1/16 keeps N(0,1) values well inside the
# format's range; the peaky keys (x8) take 1/8
FP8_SCALES = {"long_gqa8_d128_ctx128k_peaky": (1 / 8, 1 / 16)}


def to_fp8(case: Case, k_scale: float = 1 / 16, v_scale: float = 1 / 16) -> Case:
    """The same call over an E4M3 cache: K and V (bf16 values) divided by their scale and rounded
    to the nearest E4M3 value; q, lengths and page table unchanged."""
    def enc(bits, scale):
        out = np.empty(bits.shape, np.uint8)
        src, dst = bits.reshape(-1), out.reshape(-1)
        step = 1 << 22
        for i in range(0, src.size, step):
            dst[i:i + step] = f32_to_e4m3_bytes(bf16_bits_to_f32(src[i:i + step]) / np.float32(scale))
        return out
    return dataclasses.replace(case, name="fp8_" + case.name, k=enc(case.k, k_scale),
                               v=enc(case.v, v_scale), kv="fp8", k_scale=float(np.float32(k_scale)),
                               v_scale=float(np.float32(v_scale)))


def with_queries(case: Case, M: int, seed: int = 1000) -> Case:
    """The same cache with M query tokens per sequence (multi-query decode): q [B, M, Hq, D]
    drawn like q (seeded N(0,1) bf16) from default_rng(seed)."""
    rng = np.random.default_rng(seed)
    return dataclasses.replace(case, name=f"{case.name}_m{M}", q=_normal_bf16(rng, (case.B, M, case.Hq, case.D)),
                               M=M)


def make(name: str, seed: int = 0, kv: str = "bf16") -> Case:
    """A named workload; kv="fp8" gives its E4M3-cache form (see to_fp8)."""
    case = WORKLOADS[name](seed)
    if kv == "fp8":
        return to_fp8(case, *FP8_SCALES.get(name, (1 / 16, 1 / 16)))
    if kv != "bf16":
        raise ValueError(f"unknown cache type {kv!r}")
    return case
