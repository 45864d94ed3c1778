"""Shared helpers of the GPU parity tests (imported by the test modules)."""
from __future__ import annotations

import functools
import sys
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import workloads
from oracle import paged_ref as ref

# fp16 output tolerance: every element within ATOL of the fp64 oracle, and the
# relative error within RTOL wherever |ref| >= ATOL / RTOL (the two bounds
# meet there; below it the fp16 spacing alone can exceed RTOL).
ATOL = 2e-3
RTOL = 1e-2
REL_FLOOR = ATOL / RTOL
# fp32 split partials (no fp16 rounding): fp32 accumulation over at most a few
# thousand terms of magnitude <= 4.4 stays far below this.
PARTIAL_ATOL = 2e-4

DEV = "cuda:0"

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def say(msg: str):
    print(msg, file=sys.stderr, flush=True)


@functools.lru_cache(maxsize=None)
def case(name: str):
    """Cached generator call by name: 'tiny', 'qwen', 'sweep:B:ctx', 'skewed',
    'long:B:ctx'; a '+fp32' suffix ('qwen+fp32', 'sweep:32:4096+fp32',
    'long:1:32768+fp32') draws the values as fp32 normals rounded to fp16,
    tails uncut."""
    untr = name.endswith("+fp32")
    parts = name[:-5].split(":") if untr else name.split(":")
    if parts[0] == "tiny":
        return workloads.tiny_case()
    if parts[0] == "qwen":
        return workloads.qwen_case(untruncated=untr)
    if parts[0] == "sweep":
        return workloads.sweep_case(int(parts[1]), int(parts[2]), untruncated=untr)
    if parts[0] == "skewed":
        return workloads.skewed_case()
    if parts[0] == "long":
        return workloads.long_case(int(parts[1]), int(parts[2]), untruncated=untr)
    raise KeyError(name)


def to_gpu(c, device=DEV):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return SimpleNamespace(q=t(c.q), k_pool=t(c.k_pool), v_pool=t(c.v_pool),
                           bt=t(c.block_tables), ctx=t(c.context_lens), k_new=t(c.k_new),
                           v_new=t(c.v_new), slots=t(c.slot_mapping))


def host64(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def check_fp16(got: torch.Tensor, want: np.ndarray, label: str = "", rows=None):
    """Assert the fp16 GPU result is within tolerance of the fp64 oracle.
    ``rows`` restricts the comparison to some sequences (first axis)."""
    g = host64(got)
    w = np.asarray(want, dtype=np.float64)
    if rows is not None:
        g, w = g[rows], w[rows]
    assert np.all(np.isfinite(g)), f"{label}: non-finite output"
    err = np.abs(g - w)
    max_abs = float(err.max()) if err.size else 0.0
    big = np.abs(w) >= REL_FLOOR
    max_rel = float((err[big] / np.abs(w[big])).max()) if big.any() else 0.0
    assert max_abs <= ATOL, f"{label}: max abs err {max_abs:.3e} > {ATOL}"
    assert max_rel <= RTOL, f"{label}: max rel err {max_rel:.3e} > {RTOL} (|ref| >= {REL_FLOOR})"
    return max_abs, max_rel


def oracle_decode(c, seqs=None):
    return ref.paged_attention_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                                      c.scale, return_lse=True, seqs=seqs)


@functools.lru_cache(maxsize=None)
def oracle_full(name: str, appended: bool = False):
    """(out, lse) of the fp64 oracle over every sequence of a named workload,
    over its pools as generated or after the step's append of each
    sequence's new token; cached, since several tests compare the whole
    skewed batch (1.77 GB of K/V) against it."""
    c = case(name)
    if appended:
        kp, vp = ref.kv_cache_append(c.k_pool, c.v_pool, c.k_new, c.v_new, c.slot_mapping)
    else:
        kp, vp = c.k_pool, c.v_pool
    return ref.paged_attention_decode(c.q, kp, vp, c.block_tables, c.context_lens, c.scale,
                                      return_lse=True)
