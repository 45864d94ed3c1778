"""Seeded synthetic inputs for paged KV-cache decode.

This module only draws inputs: context lengths, block tables, fp16 K/V pools,
queries, the new tokens' K/V and their slot mapping.  It holds none of the
attention arithmetic; the oracle and the HIP path both consume what it returns.

Recipe:
* ``numpy.random.default_rng(seed)`` (PCG64).  Draw order: lengths, block
  tables, K pool, V pool, q, k_new, v_new.
* Values are N(0,1) in fp16, drawn by inverse-CDF sampling: each raw 64-bit
  PCG64 word gives four 16-bit indices i, and i maps to the standard normal
  quantile at probability (i + 1/2) / 65536, rounded to fp16 (nearest even).
  (Drawing fp32 normals and converting them is ~20x slower on the host and
  the 1 GB pools of the skewed workload made that the bottleneck of the
  tests.)  The tails are cut at |x| = 4.33, which changes nothing the tests
  rely on.  q of the long-context workload is then multiplied by 4 (exact).
* Block tables: ``rng.permutation(num_blocks)``; each sequence in turn takes
  the next ceil(ctx / block_size) ids; unused table entries are -1.
* Pool slots that no sequence attends (the tail of each last block, and
  unused blocks) hold fp16 NaN (0x7E00), so a kernel that lets a masked
  position contribute through a multiply by zero produces NaN.
* The new token of sequence b is appended at logical position ctx_b - 1:
  ``slot = table[b, (ctx_b-1) // bs] * bs + (ctx_b-1) % bs``.
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

NAN16 = np.uint16(0x7E00)


@dataclass
class DecodeCase:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    num_blocks: int
    scale: float
    context_lens: np.ndarray          # int32 [B]
    block_tables: np.ndarray          # int32 [B, max_blocks_per_seq], -1 pad
    k_pool: np.ndarray                # fp16 [NB, bs, Hkv, D]
    v_pool: np.ndarray                # fp16 [NB, bs, Hkv, D]
    q: np.ndarray                     # fp16 [B, Hq, D]
    k_new: np.ndarray                 # fp16 [B, Hkv, D]
    v_new: np.ndarray                 # fp16 [B, Hkv, D]
    slot_mapping: np.ndarray          # int64 [B]
    partition_size: Optional[int] = None
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    def max_partitions(self, partition_size: Optional[int] = None) -> int:
        P = partition_size or self.partition_size
        return -(-self.max_blocks_per_seq * self.block_size // P)

    def kv_bytes(self) -> int:
        """K and V bytes of the attended positions (fp16)."""
        return int(self.context_lens.astype(np.int64).sum()) * self.Hkv * self.D * 2 * 2

    def qo_bytes(self) -> int:
        """q read plus out written (fp16)."""
        return self.B * self.Hq * self.D * 2 * 2


_QUANTILES16 = None


def _quantile_table() -> np.ndarray:
    global _QUANTILES16
    if _QUANTILES16 is None:
        import scipy.special
        probs = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        _QUANTILES16 = scipy.special.ndtri(probs).astype(np.float16)
    return _QUANTILES16


_POOL = None


def _normal16(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    """N(0,1) fp16 values by inverse-CDF lookup of raw 16-bit draws.  The raw
    words are drawn in order from the one stream; the lookups of large arrays
    run on a few threads (the result does not depend on the thread count)."""
    global _POOL
    n = int(np.prod(shape))
    table = _quantile_table()
    out = np.empty(n, dtype=np.float16)
    if n <= chunk:
        idx = rng.bit_generator.random_raw((n + 3) // 4).view(np.uint16)[:n]
        out[:] = table[idx]
        return out.reshape(shape)
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max(1, min(8, len(os.sched_getaffinity(0)))))
    futs = []
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        idx = rng.bit_generator.random_raw((hi - lo + 3) // 4).view(np.uint16)[: hi - lo]
        futs.append(_POOL.submit(np.take, table, idx, 0, out[lo:hi]))
    for f in futs:
        f.result()
    return out.reshape(shape)


def _tables(rng, lens, block_size, num_blocks, max_blocks=None):
    need = [-(-int(n) // block_size) for n in lens]
    if sum(need) > num_blocks:
        raise ValueError("pool too small for the context lengths")
    maxb = max(max(need), 1) if max_blocks is None else max_blocks
    perm = rng.permutation(num_blocks).astype(np.int32)
    bt = np.full((len(lens), maxb), -1, dtype=np.int32)
    cur = 0
    for b, k in enumerate(need):
        bt[b, :k] = perm[cur:cur + k]
        cur += k
    return bt


def _poison_unattended(pool, lens, bt, block_size):
    """NaN in every slot that no sequence attends."""
    nb = pool.shape[0]
    used = np.zeros(nb, dtype=bool)
    view = pool.view(np.uint16)
    for b, n in enumerate(lens):
        n = int(n)
        k = -(-n // block_size)
        used[bt[b, :k]] = True
        tail = n - (k - 1) * block_size if k else 0
        if k and tail < block_size:
            view[bt[b, k - 1], tail:] = NAN16
    view[~used] = NAN16


def _normal16_fp32(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) fp16 values as fp32 standard normals rounded to fp16 (nearest
    even): no cut on the tails, slower on the host than _normal16."""
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


def make_case(name, *, B, Hq, Hkv, D, block_size, lens, num_blocks, seed, rng,
              scale=None, q_mult=1.0, partition_size=None, max_blocks=None,
              poison=True, untruncated=False) -> DecodeCase:
    """untruncated: draw values as fp32 normals rounded to fp16 instead of
    the inverse-CDF table (whose tails stop at |x| = 4.33)."""
    draw = (lambda shape: _normal16_fp32(rng, shape)) if untruncated else \
        (lambda shape: _normal16(rng, shape))
    lens = np.asarray(lens, dtype=np.int32)
    bt = _tables(rng, lens, block_size, num_blocks, max_blocks)
    shape = (num_blocks, block_size, Hkv, D)
    k_pool = draw(shape)
    v_pool = draw(shape)
    q = draw((B, Hq, D))
    if q_mult != 1.0:
        q = (q.astype(np.float32) * np.float32(q_mult)).astype(np.float16)
    k_new = draw((B, Hkv, D))
    v_new = draw((B, Hkv, D))
    if poison:
        _poison_unattended(k_pool, lens, bt, block_size)
        _poison_unattended(v_pool, lens, bt, block_size)
    slots = np.full(B, -1, dtype=np.int64)
    for b, n in enumerate(lens):
        if n > 0:
            pos = int(n) - 1
            slots[b] = int(bt[b, pos // block_size]) * block_size + pos % block_size
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return DecodeCase(name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=block_size,
                      num_blocks=num_blocks, scale=float(scale), context_lens=lens,
                      block_tables=bt, k_pool=k_pool, v_pool=v_pool, q=q,
                      k_new=k_new, v_new=v_new, slot_mapping=slots,
                      partition_size=partition_size, seed=seed)


# ---- the five workloads -------------------------------------------------

def tiny_case(seed: int = 1000) -> DecodeCase:
    """B=2, Hq=2, Hkv=1, D=64, bs=16, ctx {5, 37}, 8-block pool."""
    rng = np.random.default_rng(seed)
    lens = np.array([5, 37], dtype=np.int32)
    return make_case("tiny", B=2, Hq=2, Hkv=1, D=64, block_size=16, lens=lens,
                     num_blocks=8, seed=seed, rng=rng, scale=1.0 / 8.0,
                     max_blocks=4, partition_size=16)


def qwen_case(seed: int = 2000, untruncated: bool = False) -> DecodeCase:
    """Qwen2.5-0.5B attention shape: B=8, Hq=14, Hkv=2, D=64, bs=16,
    ctx ~ U{512..4096}, 4096-block pool."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(512, 4097, size=8).astype(np.int32)
    return make_case("qwen", B=8, Hq=14, Hkv=2, D=64, block_size=16, lens=lens,
                     num_blocks=4096, seed=seed, rng=rng, max_blocks=256,
                     partition_size=512, untruncated=untruncated)


SWEEP_B = (1, 8, 32)
SWEEP_CTX = (128, 512, 1024, 2048, 4096)
# Larger points on the same head configuration (trend past the sweep's corner)
EXTRA_POINTS = ((64, 4096), (128, 4096), (32, 8192), (64, 8192), (128, 8192), (32, 16384),
                (256, 8192))


def sweep_case(B: int, ctx: int, seed: Optional[int] = None,
               partition_size: int = 512, untruncated: bool = False) -> DecodeCase:
    """Batch x context sweep point: Hq=14, Hkv=2, D=64, bs=16, equal lengths."""
    if seed is None:
        seed = 3000 + 5 * SWEEP_B.index(B) + SWEEP_CTX.index(ctx)
    rng = np.random.default_rng(seed)
    lens = np.full(B, ctx, dtype=np.int32)
    nb = B * (-(-ctx // 16))
    return make_case(f"sweep_B{B}_ctx{ctx}", B=B, Hq=14, Hkv=2, D=64,
                     block_size=16, lens=lens, num_blocks=nb, seed=seed, rng=rng,
                     partition_size=partition_size, untruncated=untruncated)


def extra_case(B: int, ctx: int, partition_size: int = 512) -> DecodeCase:
    """A point of EXTRA_POINTS: the sweep's shapes at a larger batch or context."""
    seed = 3100 + EXTRA_POINTS.index((B, ctx))
    return sweep_case(B, ctx, seed=seed, partition_size=partition_size)


def skewed_lengths(rng, B=256, median=1024, sigma=1.0, lo=16, hi=32768):
    x = np.exp(rng.normal(math.log(median), sigma, size=B))
    return np.clip(np.rint(x), lo, hi).astype(np.int32)


def skewed_case(seed: int = 4000, partition_size: int = 512) -> DecodeCase:
    """B=256, Hq=32, Hkv=8, D=128, bs=16, lognormal lengths (median 1024,
    sigma 1, clipped to [16, 32768]); pool = total blocks + 10%."""
    rng = np.random.default_rng(seed)
    lens = skewed_lengths(rng)
    need = int(sum(-(-int(n) // 16) for n in lens))
    nb = int(math.ceil(1.1 * need))
    return make_case("skewed", B=256, Hq=32, Hkv=8, D=128, block_size=16,
                     lens=lens, num_blocks=nb, seed=seed, rng=rng,
                     max_blocks=32768 // 16, partition_size=partition_size)


LONG_POINTS = ((1, 32768), (1, 131072), (4, 32768), (4, 131072))


def long_case(B: int, ctx: int, seed: Optional[int] = None,
              partition_size: int = 512, untruncated: bool = False) -> DecodeCase:
    """Long-context split-K point: Hq=14, Hkv=2, D=64, bs=32, q x4."""
    if seed is None:
        seed = 5000 + LONG_POINTS.index((B, ctx))
    rng = np.random.default_rng(seed)
    lens = np.full(B, ctx, dtype=np.int32)
    nb = B * (-(-ctx // 32))
    return make_case(f"long_B{B}_ctx{ctx}", B=B, Hq=14, Hkv=2, D=64,
                     block_size=32, lens=lens, num_blocks=nb, seed=seed, rng=rng,
                     q_mult=4.0, partition_size=partition_size, untruncated=untruncated)


def custom_case(name, *, B, Hq, Hkv, D, block_size, lens, seed, num_blocks=None,
                max_blocks=None, partition_size=None, q_mult=1.0, scale=None,
                poison=True) -> DecodeCase:
    """Any shape, for edge cases (ragged tails, ctx 0/1, many partitions)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    need = int(sum(-(-int(n) // block_size) for n in lens))
    if num_blocks is None:
        num_blocks = max(need + 3, 1)
    return make_case(name, B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=block_size,
                     lens=lens, num_blocks=num_blocks, seed=seed, rng=rng,
                     scale=scale, q_mult=q_mult, partition_size=partition_size,
                     max_blocks=max_blocks, poison=poison)


# ---- chunked prefill -------------------------------------------------------

@dataclass
class PrefillCase:
    """A chunk of new tokens per sequence over a paged cache.

    Sequence b's chunk is rows query_start[b] .. query_start[b+1]-1 of q; it
    holds the last n_b of the sequence's context_lens[b] positions.  k_pool /
    v_pool hold every attended position including the chunk's; k_chunk /
    v_chunk are the chunk's rows (what a multi-token append writes) and
    chunk_slots their slots, so a test can poison those slots, append, then
    attend."""
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    num_blocks: int
    scale: float
    context_lens: np.ndarray          # int32 [B]
    query_start: np.ndarray           # int32 [B + 1]
    block_tables: np.ndarray          # int32 [B, max_blocks_per_seq]
    k_pool: np.ndarray                # fp16 [NB, bs, Hkv, D]
    v_pool: np.ndarray
    q: np.ndarray                     # fp16 [total_q, Hq, D]
    k_chunk: np.ndarray               # fp16 [total_q, Hkv, D]
    v_chunk: np.ndarray
    chunk_slots: np.ndarray           # int64 [total_q]
    seed: int = 0

    @property
    def total_q(self) -> int:
        return int(self.query_start[-1])

    @property
    def chunk_lens(self) -> np.ndarray:
        return np.diff(self.query_start).astype(np.int32)

    @property
    def max_q(self) -> int:
        return int(self.chunk_lens.max()) if self.B else 0


def prefill_case(name, *, Hq, Hkv, D, block_size, ctx, chunk, seed, q_mult=1.0,
                 scale=None, num_blocks=None) -> PrefillCase:
    """Pool and tables as ``custom_case`` for context lengths ``ctx``; then
    ``chunk[b]`` query rows per sequence (drawn after everything else)."""
    ctx = np.asarray(ctx, dtype=np.int32)
    chunk = np.asarray(chunk, dtype=np.int32)
    B = len(ctx)
    base = custom_case(name, B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=block_size, lens=ctx,
                       seed=seed, q_mult=q_mult, scale=scale, num_blocks=num_blocks)
    rng = np.random.default_rng(seed + 7919)
    qs = np.zeros(B + 1, dtype=np.int32)
    qs[1:] = np.cumsum(chunk)
    q = _normal16(rng, (int(qs[-1]), Hq, D))
    if q_mult != 1.0:
        q = (q.astype(np.float32) * np.float32(q_mult)).astype(np.float16)
    slots = []
    for b in range(B):
        for i in range(int(chunk[b])):
            pos = int(ctx[b]) - int(chunk[b]) + i
            if pos < 0:
                slots.append(-1)
            else:
                slots.append(int(base.block_tables[b, pos // block_size]) * block_size
                             + pos % block_size)
    slots = np.asarray(slots, dtype=np.int64)
    blk = np.where(slots >= 0, slots // block_size, 0)
    off = np.where(slots >= 0, slots % block_size, 0)
    k_chunk = base.k_pool[blk, off].copy()
    v_chunk = base.v_pool[blk, off].copy()
    return PrefillCase(name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=block_size,
                       num_blocks=base.num_blocks, scale=base.scale, context_lens=ctx,
                       query_start=qs, block_tables=base.block_tables, k_pool=base.k_pool,
                       v_pool=base.v_pool, q=q, k_chunk=k_chunk, v_chunk=v_chunk,
                       chunk_slots=slots, seed=seed)


# ---- 8-bit cache -------------------------------------------------------------

def q8_pools(case, seed: Optional[int] = None):
    """Random 8-bit K/V pools with the case's shapes: int8 codes uniform in
    [-127, 127] with one +-127 per row (as a quantised row always has), and
    per-(token, head) fp32 scales uniform in [2, 4.5] / 127 (the amax of
    N(0,1) rows of 64-128 values).  Rows no sequence attends (NaN in the
    case's fp16 pools) get a NaN scale.  Codes are returned [NB, bs, Hkv, D]
    and scales [NB, bs, Hkv] (the oracle's order); the library's layouts are
    head-major, [NB, Hkv, bs, D] and [NB, Hkv, bs].
    Returns (k_codes, v_codes, k_scales, v_scales)."""
    rng = np.random.default_rng(case.seed + 13 if seed is None else seed)
    NB, bs, Hkv, D = case.k_pool.shape
    unattended = np.isnan(case.k_pool[..., 0].astype(np.float32))

    def pool():
        codes = rng.integers(-127, 128, (NB, bs, Hkv, D), dtype=np.int8)
        top = rng.integers(0, D, (NB, bs, Hkv, 1))
        sign = np.where(rng.random((NB, bs, Hkv, 1)) < 0.5, -127, 127).astype(np.int8)
        np.put_along_axis(codes, top, sign, axis=-1)
        scales = (rng.uniform(2.0, 4.5, (NB, bs, Hkv)) / 127.0).astype(np.float32)
        scales[unattended] = np.nan
        return codes, scales

    kc, ks = pool()
    vc, vs = pool()
    return kc, vc, ks, vs
