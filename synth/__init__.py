"""Seeded synthetic inputs for DiffQKV attention.

This module is the one piece shared by the fp64 oracle's tests and by the GPU
path's tests and benchmark.  It draws random numbers and lays them out; it
holds none of the attention arithmetic.

Every tensor comes from its own PCG64 streams, keyed by ``(seed, stream id,
block)`` for consecutive blocks of 2^24 elements, so two layouts that share a
tensor shape (for example the V cache of the asymmetric layout and of its
symmetric twin) receive identical bytes, and a tensor of another shape (K, Q)
is drawn from the same streams at its own size.  Blocks are filled by a pool
of threads; the values do not depend on how many.

bf16 tensors are returned as their raw ``uint16`` bit patterns, obtained from
float32 normals by round-to-nearest-even; :func:`bf16_bits_to_f32` widens them
back exactly.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# Stream ids: one per tensor role.
S_Q, S_K, S_V, S_KNEW, S_VNEW, S_LEN, S_OUTLIER = 1, 2, 3, 4, 5, 6, 7
S_H, S_WGATE, S_WUP, S_WDOWN = 8, 9, 10, 11

BF16_NAN = np.uint16(0x7FC0)
_BLOCK = 1 << 24  # elements per generator block (part of the values' definition)
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _rng(seed: int, stream: int, block: int | None = None) -> np.random.Generator:
    key = [int(seed), int(stream)] if block is None else [int(seed), int(stream), int(block)]
    return np.random.default_rng(key)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even; returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(seed: int, stream: int, shape, dtype: str) -> np.ndarray:
    """N(0,1) samples of ``shape``: float32 array, or uint16 bf16 bits.

    Element e belongs to block e // 2^24, whose samples come from the
    generator keyed (seed, stream, block); blocks are filled in parallel
    (numpy's generators and array arithmetic release the interpreter lock),
    so the values depend on the seed, the stream and the shape only.
    """
    n = int(np.prod(shape)) if len(shape) else 1
    if dtype == "f32":
        out = np.empty(n, dtype=np.float32)
    elif dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
    else:
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")

    def fill(blk: int) -> None:
        s = blk * _BLOCK
        e = min(n, s + _BLOCK)
        x = _rng(seed, stream, blk).standard_normal(e - s, dtype=np.float32)
        out[s:e] = x if dtype == "f32" else f32_to_bf16_bits(x)

    n_blocks = -(-n // _BLOCK)
    if n_blocks <= 1:
        for blk in range(n_blocks):
            fill(blk)
    else:
        with ThreadPoolExecutor(max_workers=min(_THREADS, n_blocks)) as ex:
            list(ex.map(fill, range(n_blocks)))
    return out.reshape(shape)


def ragged_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Per-sequence lengths drawn uniformly from the integers lo..hi inclusive."""
    return _rng(seed, S_LEN).integers(lo, hi + 1, size=batch).astype(np.int32)


def outlier_channels(seed: int, n_heads: int, d: int, frac: float = 0.01):
    """ceil(frac * n_heads * d) distinct (head, channel) pairs chosen by seed."""
    count = int(math.ceil(frac * n_heads * d))
    flat = _rng(seed, S_OUTLIER).choice(n_heads * d, size=count, replace=False)
    return [(int(f) // d, int(f) % d) for f in np.sort(flat)]


@dataclass
class DecodeCase:
    """Host-side inputs of one decode (or prefill) call.

    Layouts: q ``[B][n_q][d_k]`` for decode, ``[B][t_new][n_q][d_k]`` for
    prefill; caches head-major ``K[B][n_k][l_cap][d_k]``,
    ``V[B][n_v][l_cap][d_v]``; ``ctx_len[B]`` rows attended per sequence.
    Arrays are float32 (dtype ``f32``) or uint16 bf16 bits (``bf16``).
    """

    dtype: str
    n_q: int
    n_k: int
    n_v: int
    d_k: int
    d_v: int
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    ctx_len: np.ndarray
    scale: float
    t_new: int = 0
    outliers: list = field(default_factory=list)

    @property
    def batch(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def l_cap(self) -> int:
        return int(self.k_cache.shape[2])

    def widened(self):
        """(q, K, V) as float32 arrays (exact for bf16 inputs)."""
        if self.dtype == "f32":
            return self.q, self.k_cache, self.v_cache
        return (bf16_bits_to_f32(self.q), bf16_bits_to_f32(self.k_cache),
                bf16_bits_to_f32(self.v_cache))


def _fill_tail(cache: np.ndarray, lengths: np.ndarray, dtype: str) -> None:
    """Poison cache rows at or past each sequence's length with NaN."""
    nan = BF16_NAN if dtype == "bf16" else np.float32("nan")
    for b, L in enumerate(lengths):
        cache[b, :, int(L):, :] = nan


def _apply_outliers(k: np.ndarray, pairs, factor: float, dtype: str) -> None:
    for h, ch in pairs:
        if dtype == "bf16":
            col = bf16_bits_to_f32(k[:, h, :, ch]) * np.float32(factor)
            k[:, h, :, ch] = f32_to_bf16_bits(col)
        else:
            k[:, h, :, ch] *= np.float32(factor)


def make_case(seed: int, *, dtype: str, batch: int, n_q: int, n_k: int,
              n_v: int, d_k: int, d_v: int, ctx_len, l_cap: int | None = None,
              t_new: int = 0, outlier_frac: float = 0.0,
              outlier_factor: float = 8.0, poison_tail: bool = False,
              scale: float | None = None) -> DecodeCase:
    """Build one seeded case.

    ``ctx_len`` is an int or a length-``batch`` sequence of rows attended.
    ``t_new`` > 0 makes a prefill case (q holds ``t_new`` rows per sequence).
    ``outlier_frac`` > 0 multiplies that fraction of K's (head, channel)
    pairs by ``outlier_factor`` for every token.  ``poison_tail`` fills cache
    rows past each length with NaN so that any read of them shows up.
    """
    lengths = np.broadcast_to(np.asarray(ctx_len, dtype=np.int32), (batch,)).copy()
    if l_cap is None:
        l_cap = int(lengths.max()) if batch else 1
    if t_new:
        q = normal(seed, S_Q, (batch, t_new, n_q, d_k), dtype)
    else:
        q = normal(seed, S_Q, (batch, n_q, d_k), dtype)
    k = normal(seed, S_K, (batch, n_k, l_cap, d_k), dtype)
    v = normal(seed, S_V, (batch, n_v, l_cap, d_v), dtype)
    pairs = outlier_channels(seed, n_k, d_k, outlier_frac) if outlier_frac > 0 else []
    if pairs:
        _apply_outliers(k, pairs, outlier_factor, dtype)
    if poison_tail:
        _fill_tail(k, lengths, dtype)
        _fill_tail(v, lengths, dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    return DecodeCase(dtype, n_q, n_k, n_v, d_k, d_v, q, k, v, lengths,
                      float(scale), t_new, pairs)


def new_rows(seed: int, *, dtype: str, batch: int, t_new: int, n_k: int,
             n_v: int, d_k: int, d_v: int):
    """Token-major rows to append: ``k_new[B][t_new][n_k][d_k]``,
    ``v_new[B][t_new][n_v][d_v]``."""
    k_new = normal(seed, S_KNEW, (batch, t_new, n_k, d_k), dtype)
    v_new = normal(seed, S_VNEW, (batch, t_new, n_v, d_v), dtype)
    return k_new, v_new


@dataclass
class AugQCase:
    """Inputs of the augmented-Q projection: hidden states h [M][d_m] and
    weights in (out, in) layout, W_gate / W_up [d_i][d_m], W_down
    [d_out][d_i]; float32 arrays or uint16 bf16 bits."""

    dtype: str
    h: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray

    def widened(self):
        if self.dtype == "f32":
            return self.h, self.w_gate, self.w_up, self.w_down
        return tuple(bf16_bits_to_f32(x) for x in (self.h, self.w_gate, self.w_up, self.w_down))


def _scaled(seed, stream, shape, fan_in, dtype):
    x = normal(seed, stream, shape, "f32") * np.float32(1.0 / math.sqrt(fan_in))
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def make_augq(seed: int, *, M: int, d_m: int, d_i: int, d_out: int,
              dtype: str = "bf16") -> AugQCase:
    """Seeded augmented-Q inputs: h ~ N(0, 1); weights ~ N(0, 1/fan_in), the
    usual initialisation scale, so the intermediate and output stay O(1)."""
    h = normal(seed, S_H, (M, d_m), dtype)
    return AugQCase(dtype, h, _scaled(seed, S_WGATE, (d_i, d_m), d_m, dtype),
                    _scaled(seed, S_WUP, (d_i, d_m), d_m, dtype),
                    _scaled(seed, S_WDOWN, (d_out, d_i), d_i, dtype))


# The SIGMA-1.5B augmented-Q shape (architecture page, Table 14): hidden
# 2048, augmented intermediate 3072, 32 query heads of 64 dimensions.
AUGQ_SIGMA15B = dict(d_m=2048, d_i=3072, d_out=32 * 64)


# ---------------------------------------------------------------------------
# The workloads measured and parity-tested.  Each entry gives the seed and the
# keyword arguments of make_case (lengths may be drawn from the seed).

def workload(name: str) -> dict:
    """Keyword arguments of :func:`make_case` for a named workload."""
    if name == "tiny_f32":
        return dict(seed=1, dtype="f32", batch=1, n_q=4, n_k=1, n_v=4, d_k=32,
                    d_v=64, ctx_len=256)
    if name == "decode32k_asym":
        return dict(seed=2, dtype="bf16", batch=1, n_q=16, n_k=4, n_v=16,
                    d_k=64, d_v=128, ctx_len=32768)
    if name == "decode32k_sym":
        return dict(seed=2, dtype="bf16", batch=1, n_q=16, n_k=16, n_v=16,
                    d_k=128, d_v=128, ctx_len=32768)
    if name == "ragged16":
        old = ragged_lengths(3, 16, 4096, 32768)
        return dict(seed=3, dtype="bf16", batch=16, n_q=16, n_k=4, n_v=16,
                    d_k=64, d_v=128, ctx_len=old, l_cap=32769)
    if name.startswith("decode64k_"):
        shape = {"decode64k_dk64": (4, 16, 64, 128),
                 "decode64k_dk128": (4, 16, 128, 128),
                 "decode64k_sym": (16, 16, 128, 128)}[name]
        n_k, n_v, d_k, d_v = shape
        return dict(seed=4, dtype="bf16", batch=4, n_q=16, n_k=n_k, n_v=n_v,
                    d_k=d_k, d_v=d_v, ctx_len=65536, outlier_frac=0.01,
                    outlier_factor=8.0)
    if name.startswith("ket_"):
        # The pages' efficiency comparison: SIGMA-1.5B attention (32 query,
        # 4 key, 16 value heads, head dimension 64) against their standard
        # GQA model (16 key and 16 value heads), one sequence, at a prefix.
        _, model, prefix = name.split("_")
        n_k = {"sigma": 4, "std": 16}[model]
        return dict(seed=6, dtype="bf16", batch=1, n_q=32, n_k=n_k, n_v=16, d_k=64,
                    d_v=64, ctx_len=int(prefix))
    if name == "prefill2k_on_30k":
        return dict(seed=5, dtype="bf16", batch=1, n_q=16, n_k=4, n_v=16,
                    d_k=64, d_v=128, ctx_len=32768, t_new=2048)
    raise KeyError(name)


KET_PREFIXES = (2048, 4096, 16384, 32768)

WORKLOADS = ("tiny_f32", "decode32k_asym", "decode32k_sym", "ragged16",
             "decode64k_dk64", "decode64k_dk128", "decode64k_sym",
             "prefill2k_on_30k") + tuple(
                 f"ket_{m}_{p}" for p in KET_PREFIXES for m in ("sigma", "std"))
