"""paged_attention_decode_split + split_reduce on the GPU against the oracle
(partials and merged output), and against the unsplit kernel."""
import numpy as np
import pytest
import torch

import paged_kv_decode_cache_amd as pkv
import workloads
from oracle import paged_ref as ref
from gpu_common import (PARTIAL_ATOL, case, check_fp16, host64, needs_gpu, oracle_decode,
                        oracle_full, say, to_gpu)

pytestmark = [pytest.mark.gpu, needs_gpu]


def _split_reduce(g, c, P, Pm=None, launch=None):
    po, pl = pkv.paged_attention_decode_split(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, c.scale,
                                              P, max_partitions=Pm, launch=launch)
    out, lse = pkv.split_reduce(po, pl, g.ctx, P, want_lse=True)
    return po, pl, out, lse


def _check_lse(got, want, label, rows=None):
    g = host64(got)
    w = np.asarray(want, dtype=np.float64)
    if rows is not None:
        g, w = g[rows], w[rows]
    fin = np.isfinite(w)
    assert np.array_equal(np.isneginf(g), np.isneginf(w)), f"{label}: -inf pattern differs"
    if fin.any():
        err = float(np.abs(g[fin] - w[fin]).max())
        assert err <= PARTIAL_ATOL, f"{label}: lse err {err:.3e}"


LONG = [f"long:{B}:{ctx}" for B, ctx in workloads.LONG_POINTS]


@pytest.mark.parametrize("name", LONG)
def test_long_context_split_matches_oracle_and_unsplit(name):
    c = case(name)
    P = 512
    say(f"split {name}: P={P}")
    g = to_gpu(c)
    po, pl, out, lse = _split_reduce(g, c, P)
    unsplit = pkv.paged_attention_decode(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, c.scale)
    torch.cuda.synchronize()
    want, want_lse = oracle_decode(c)
    check_fp16(out, want, name + " split")
    _check_lse(lse, want_lse, name)
    d = (out.float() - unsplit.float()).abs().max().item()
    assert d <= 2e-3, f"split vs unsplit differ by {d}"


@pytest.mark.parametrize("name,P", [("tiny", 16), ("qwen", 512), ("qwen", 64),
                                    ("sweep:32:4096", 256), ("sweep:1:128", 512),
                                    ("sweep:8:1024", 16)])
def test_split_partials_match_oracle(name, P):
    c = case(name)
    say(f"split partials {name}: P={P}")
    g = to_gpu(c)
    Pm = c.max_partitions(P)
    po, pl, out, lse = _split_reduce(g, c, P, Pm)
    torch.cuda.synchronize()
    wpo, wpl = ref.paged_attention_decode_split(c.q, c.k_pool, c.v_pool, c.block_tables,
                                                c.context_lens, c.scale, P, Pm)
    gpl = host64(pl)
    gpo = host64(po)
    assert np.array_equal(np.isneginf(gpl), np.isneginf(wpl))
    valid = np.isfinite(wpl)
    assert float(np.abs(gpl[valid] - wpl[valid]).max()) <= PARTIAL_ATOL
    assert float(np.abs(gpo[valid] - wpo[valid]).max()) <= PARTIAL_ATOL
    want, want_lse = oracle_decode(c)
    check_fp16(out, want, f"{name} P={P}")
    _check_lse(lse, want_lse, name)


@pytest.mark.parametrize("grid", ["auto", "compact"])
def test_skewed_split_full(grid):
    """The skewed batch (B=256, lognormal lengths, ragged partitions) on the
    default grid and the compact grid, every sequence against the oracle."""
    c = case("skewed")
    P = 512
    say(f"split skewed P={P} grid={grid} (all {c.B} sequences)")
    g = to_gpu(c)
    po, pl, out, lse = _split_reduce(g, c, P, launch=dict(grid=grid))
    torch.cuda.synchronize()
    want, want_lse = oracle_full("skewed")
    check_fp16(out, want, f"skewed split {grid}")
    _check_lse(lse, want_lse, f"skewed {grid}")


def test_split_compact_grid_large_ragged_batch():
    """A ragged batch of 300 sequences (lengths 0..2000) on the compact grid:
    the two-ballot sequence search walks a prefix array with step > 1; every
    sequence against the oracle, -inf lse on every empty partition."""
    rng = np.random.default_rng(132)
    lens = rng.integers(0, 2001, 300).tolist()
    lens[0], lens[1], lens[299] = 0, 2000, 1
    c = workloads.custom_case("compact_300", B=300, Hq=14, Hkv=2, D=64, block_size=16, lens=lens,
                              seed=133)
    g = to_gpu(c)
    P = 128
    po, pl, out, lse = _split_reduce(g, c, P, launch=dict(grid="compact"))
    torch.cuda.synchronize()
    wpo, wpl = ref.paged_attention_decode_split(c.q, c.k_pool, c.v_pool, c.block_tables,
                                                c.context_lens, c.scale, P, c.max_partitions(P))
    assert np.array_equal(np.isneginf(host64(pl)), np.isneginf(wpl))
    want, want_lse = oracle_decode(c)
    check_fp16(out, want, "compact B=300")
    _check_lse(lse, want_lse, "compact B=300")


def test_partition_larger_than_context_and_spare_partitions():
    c = workloads.custom_case("spare", B=4, Hq=14, Hkv=2, D=64, block_size=32,
                              lens=[1, 31, 32, 600], seed=98, q_mult=4.0)
    g = to_gpu(c)
    for P, extra in ((1024, 0), (1024, 3), (32, 5), (64, 1)):
        Pm = c.max_partitions(P) + extra
        po, pl, out, lse = _split_reduce(g, c, P, Pm)
        torch.cuda.synchronize()
        want, want_lse = oracle_decode(c)
        check_fp16(out, want, f"spare P={P}+{extra}")
        _check_lse(lse, want_lse, f"spare P={P}")
        gpl = host64(pl)
        for b, n in enumerate(c.context_lens):
            used = -(-int(n) // P)
            assert np.all(np.isfinite(gpl[b, :, :used]))
            assert np.all(np.isneginf(gpl[b, :, used:]))


def test_split_ctx0():
    c = workloads.custom_case("sctx0", B=2, Hq=4, Hkv=1, D=128, block_size=16, lens=[0, 40],
                              seed=99)
    g = to_gpu(c)
    po, pl, out, lse = _split_reduce(g, c, 32)
    torch.cuda.synchronize()
    assert int((out[0] != 0).sum()) == 0
    assert torch.isneginf(lse[0]).all()
    want, want_lse = oracle_decode(c)
    check_fp16(out, want, "split ctx0")
    _check_lse(lse, want_lse, "split ctx0")


@pytest.mark.parametrize("waves", [1, 2, 4, 8])
@pytest.mark.parametrize("subtiles", [1, 2, 4])
@pytest.mark.parametrize("depth", [2, 4])
def test_split_every_launch_shape(waves, subtiles, depth):
    launch = dict(waves=waves, subtiles=subtiles, depth=depth)
    c = case("qwen")
    g = to_gpu(c)
    po, pl, out, lse = _split_reduce(g, c, 256, launch=launch)
    torch.cuda.synchronize()
    want, want_lse = oracle_decode(c)
    check_fp16(out, want, f"split NW={waves} NS={subtiles} DEPTH={depth}")
    _check_lse(lse, want_lse, "split shapes")
    # head_dim 128, group 16 (both parts of P in one 16x16x32 MFMA), block size 32
    c2 = workloads.custom_case("split_d128_g16", B=3, Hq=16, Hkv=1, D=128, block_size=32,
                               lens=[33, 700, 1500], seed=100)
    g2 = to_gpu(c2)
    po, pl, out2, lse2 = _split_reduce(g2, c2, 256, launch=launch)
    torch.cuda.synchronize()
    want2, want_lse2 = oracle_decode(c2)
    check_fp16(out2, want2, f"split d128 g16 NW={waves} NS={subtiles} DEPTH={depth}")


@pytest.mark.parametrize("name,P", [("tiny", 16), ("qwen", 256), ("sweep:8:1024", 64),
                                    ("long:1:32768", 512)])
def test_split_compact_grid_matches_oracle(name, P):
    """The compact grid (workgroups looping over the non-empty items) gives
    the oracle's partials, with -inf lse on every empty partition."""
    c = case(name)
    say(f"split compact {name}: P={P}")
    g = to_gpu(c)
    Pm = c.max_partitions(P) + 2
    po, pl, out, lse = _split_reduce(g, c, P, Pm, launch=dict(grid="compact"))
    torch.cuda.synchronize()
    wpo, wpl = ref.paged_attention_decode_split(c.q, c.k_pool, c.v_pool, c.block_tables,
                                                c.context_lens, c.scale, P, Pm)
    gpl = host64(pl)
    assert np.array_equal(np.isneginf(gpl), np.isneginf(wpl))
    valid = np.isfinite(wpl)
    assert float(np.abs(gpl[valid] - wpl[valid]).max()) <= PARTIAL_ATOL
    assert float(np.abs(host64(po)[valid] - wpo[valid]).max()) <= PARTIAL_ATOL
    want, want_lse = oracle_decode(c)
    check_fp16(out, want, f"compact {name}")
    _check_lse(lse, want_lse, name)


def test_split_compact_ragged_and_empty_sequences():
    c = workloads.custom_case("compact_ragged", B=7, Hq=14, Hkv=2, D=64, block_size=16,
                              lens=[0, 1, 700, 16, 0, 2049, 33], seed=102, max_blocks=160)
    g = to_gpu(c)
    po, pl, out, lse = _split_reduce(g, c, 64, launch=dict(grid="compact"))
    torch.cuda.synchronize()
    want, want_lse = oracle_decode(c)
    check_fp16(out, want, "compact ragged")
    _check_lse(lse, want_lse, "compact ragged")
    assert torch.isneginf(pl[0]).all() and torch.isneginf(pl[4]).all()


def test_split_reduce_many_rows_few_partitions():
    """Large batch, few partitions (the library's row-batched merge): B=320 at
    Hq=14 (4,480 pairs), lengths 1..600 at P=64 and P=512, and the same merge
    of the split prefill's rows is covered in tests/test_prefill_gpu.py."""
    rng = np.random.default_rng(130)
    lens = rng.integers(1, 601, 320).tolist()
    c = workloads.custom_case("many_rows", B=320, Hq=14, Hkv=2, D=64, block_size=16, lens=lens,
                              seed=131)
    g = to_gpu(c)
    want, want_lse = oracle_decode(c)
    for P in (64, 512):
        po, pl = pkv.paged_attention_decode_split(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, c.scale,
                                                  P)
        out, lse = pkv.split_reduce(po, pl, g.ctx, P, want_lse=True)
        torch.cuda.synchronize()
        check_fp16(out, want, f"many rows P={P}")
        _check_lse(lse, want_lse, f"many rows P={P}")
