"""paged_attention_decode on the GPU against the fp64 oracle, plus the
bit-exact properties of its indexing path."""
import numpy as np
import pytest
import torch

import paged_kv_decode_cache_amd as pkv
import workloads
from oracle import paged_ref as ref
from gpu_common import (DEV, case, check_fp16, needs_gpu, oracle_decode, oracle_full, say,
                        to_gpu)

pytestmark = [pytest.mark.gpu, needs_gpu]

SWEEP = [f"sweep:{B}:{ctx}" for B in workloads.SWEEP_B for ctx in workloads.SWEEP_CTX]
FULL_ORACLE = ["tiny", "qwen"] + SWEEP + ["long:1:32768", "long:1:131072", "long:4:32768"]


def _decode(g, c, launch=None):
    return pkv.paged_attention_decode(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, c.scale,
                                      launch=launch)


@pytest.mark.parametrize("name", FULL_ORACLE)
def test_decode_matches_oracle(name):
    c = case(name)
    say(f"decode {name}: B={c.B} Hq={c.Hq} Hkv={c.Hkv} D={c.D} bs={c.block_size} "
        f"ctx max {int(c.context_lens.max())}")
    g = to_gpu(c)
    out = _decode(g, c)
    torch.cuda.synchronize()
    want, _ = oracle_decode(c)
    check_fp16(out, want, name)


@pytest.mark.parametrize("name", ["skewed", "long:4:131072"])
def test_decode_matches_oracle_full_size(name):
    """Full-size launch, every sequence against the oracle."""
    c = case(name)
    say(f"decode {name} (all {c.B} sequences)")
    g = to_gpu(c)
    out = _decode(g, c)
    torch.cuda.synchronize()
    want, _ = oracle_full(name)
    check_fp16(out, want, name)
    assert torch.isfinite(out.float()).all()


def test_append_then_decode_step():
    """One decode step of the tiny workload: append each sequence's new K/V at
    position ctx-1, then attend over [0, ctx)."""
    for name in ("tiny", "qwen"):
        c = case(name)
        say(f"append+decode step {name}")
        g = to_gpu(c)
        pkv.kv_cache_append(g.k_pool, g.v_pool, g.k_new, g.v_new, g.slots)
        out = _decode(g, c)
        torch.cuda.synchronize()
        kp, vp = ref.kv_cache_append(c.k_pool, c.v_pool, c.k_new, c.v_new, c.slot_mapping)
        want = ref.paged_attention_decode(c.q, kp, vp, c.block_tables, c.context_lens, c.scale)
        check_fp16(out, want, name + " step")


def test_argmax_probe_bit_exact():
    """q = 64 e0 and one key row 64 e0, every other key 0 in dim 0: the logit
    gap is 512, exp(-512) is 0 in fp32, so the output is exactly that V row.
    The hot position sweeps over the context, one per batch row."""
    B, Hq, Hkv, D, bs, ctx = 64, 14, 2, 64, 16, 1000
    c = workloads.custom_case("probe", B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=bs,
                              lens=[ctx] * B, seed=90)
    kp = c.k_pool.copy()
    kp[..., 0] = 0.0
    q = c.q.copy()
    q[:] = 0.0
    q[..., 0] = 64.0
    hot = np.linspace(0, ctx - 1, B).astype(int)
    hot[1] = 15
    hot[2] = 16
    hot[3] = ctx - 1
    for b in range(B):
        t = int(hot[b])
        kp[c.block_tables[b, t // bs], t % bs, :, 0] = 64.0
    g = to_gpu(c)
    g.k_pool = torch.from_numpy(kp).to(DEV)
    g.q = torch.from_numpy(q).to(DEV)
    out = pkv.paged_attention_decode(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, 0.125)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(B):
        t = int(hot[b])
        for h in range(Hq):
            row = c.v_pool[c.block_tables[b, t // bs], t % bs, h // (Hq // Hkv)]
            assert np.array_equal(got[b, h].view(np.uint16), row.view(np.uint16)), (b, h, t)


def test_ctx1_returns_v_row_bit_exact():
    c = workloads.custom_case("ctx1", B=5, Hq=16, Hkv=4, D=128, block_size=32,
                              lens=[1] * 5, seed=91)
    g = to_gpu(c)
    out = _decode(g, c)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b in range(5):
        for h in range(16):
            row = c.v_pool[c.block_tables[b, 0], 0, h // 4]
            assert np.array_equal(got[b, h].view(np.uint16), row.view(np.uint16))


def test_block_permutation_bit_identical():
    c = case("qwen")
    g = to_gpu(c)
    base = _decode(g, c).cpu()
    rng = np.random.default_rng(92)
    perm = rng.permutation(c.num_blocks)
    kp = np.empty_like(c.k_pool)
    vp = np.empty_like(c.v_pool)
    kp[perm] = c.k_pool
    vp[perm] = c.v_pool
    bt = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    g2 = to_gpu(c)
    g2.k_pool = torch.from_numpy(kp).to(DEV)
    g2.v_pool = torch.from_numpy(vp).to(DEV)
    g2.bt = torch.from_numpy(bt).to(DEV)
    moved = _decode(g2, c).cpu()
    assert torch.equal(base.view(torch.int16), moved.view(torch.int16))


def test_run_to_run_deterministic():
    c = case("sweep:8:2048")
    g = to_gpu(c)
    a = _decode(g, c).cpu()
    b = _decode(g, c).cpu()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


EDGE = [
    # name, Hq, Hkv, D, bs, lens
    ("ragged_g7", 14, 2, 64, 16, [1, 2, 15, 16, 17, 31, 33, 63, 64, 65, 127, 1000]),
    ("mha_d128", 4, 4, 128, 16, [3, 77, 500]),
    ("g16", 16, 1, 64, 32, [40, 700, 1]),
    ("g4_bs64", 32, 8, 128, 64, [100, 1, 900]),
    ("g2_bs256", 4, 2, 64, 256, [255, 256, 257, 2000]),
    ("g1_d64_bs32", 3, 3, 64, 32, [5, 32, 96, 1000]),
    ("g8_d128_bs16", 8, 1, 128, 16, [16, 48, 4096]),
    ("g12_d64_bs16", 12, 1, 64, 16, [1, 100, 777]),      # 9..15 heads: padded columns
    ("g10_d128_bs32", 20, 2, 128, 32, [31, 500, 2049]),
]


@pytest.mark.parametrize("name,Hq,Hkv,D,bs,lens", EDGE, ids=[e[0] for e in EDGE])
def test_decode_edge_shapes(name, Hq, Hkv, D, bs, lens):
    c = workloads.custom_case(name, B=len(lens), Hq=Hq, Hkv=Hkv, D=D, block_size=bs,
                              lens=lens, seed=93)
    say(f"decode edge {name}")
    g = to_gpu(c)
    out = _decode(g, c)
    torch.cuda.synchronize()
    want, _ = oracle_decode(c)
    check_fp16(out, want, name)


def test_ctx0_gives_zeros():
    c = workloads.custom_case("ctx0", B=3, Hq=14, Hkv=2, D=64, block_size=16, lens=[0, 20, 0],
                              seed=94)
    g = to_gpu(c)
    out = _decode(g, c)
    torch.cuda.synchronize()
    assert int((out[0] != 0).sum()) == 0 and int((out[2] != 0).sum()) == 0
    want, _ = oracle_decode(c)
    check_fp16(out, want, "ctx0")


def test_peaked_softmax_large_outputs():
    """q x 4 (logit std 4) over short and long contexts: close to one-hot
    weights, outputs near the V extremes, the hardest case for the 2e-3 bound."""
    c = workloads.custom_case("peaked", B=6, Hq=14, Hkv=2, D=64, block_size=16,
                              lens=[2, 3, 5, 50, 700, 3000], seed=95, q_mult=4.0)
    g = to_gpu(c)
    out = _decode(g, c)
    torch.cuda.synchronize()
    want, _ = oracle_decode(c)
    check_fp16(out, want, "peaked")


@pytest.mark.parametrize("waves", [1, 2, 4, 8])
@pytest.mark.parametrize("subtiles", [1, 2, 4])
@pytest.mark.parametrize("depth", [2, 4])
def test_decode_every_launch_shape(waves, subtiles, depth):
    launch = dict(waves=waves, subtiles=subtiles, depth=depth)
    for name, D in (("qwen", 64), ("d128", 128)):
        if name == "qwen":
            c = case("qwen")
        else:
            c = workloads.custom_case("d128", B=3, Hq=32, Hkv=8, D=128, block_size=16,
                                      lens=[1, 300, 1111], seed=96)
        g = to_gpu(c)
        out = _decode(g, c, launch=launch)
        torch.cuda.synchronize()
        want, _ = oracle_decode(c)
        check_fp16(out, want, f"{name} NW={waves} NS={subtiles} DEPTH={depth}")


def test_out_of_range_block_ids_are_ignored():
    """Block ids outside [0, num_blocks) are not read; their positions drop
    out of the softmax, and the other sequences are unaffected."""
    c = workloads.custom_case("badids", B=3, Hq=14, Hkv=2, D=64, block_size=16,
                              lens=[64, 64, 100], seed=97, poison=False)
    bt = c.block_tables.copy()
    bt[1, 1] = c.num_blocks + 7          # positions 16..31 of sequence 1
    bt[1, 2] = -5                        # positions 32..47
    g = to_gpu(c)
    g.bt = torch.from_numpy(bt).to(DEV)
    out = _decode(g, c)
    torch.cuda.synchronize()
    want, _ = oracle_decode(c)
    check_fp16(out, want, "badids", rows=[0, 2])
    # sequence 1 equals attention over its positions in valid blocks only
    keep = [0, 3]
    kp = c.k_pool[c.block_tables[1, keep]]
    vp = c.v_pool[c.block_tables[1, keep]]
    w1 = ref.paged_attention_decode(c.q[1:2], kp, vp, np.array([[0, 1]], np.int32),
                                    np.array([32], np.int32), c.scale)
    check_fp16(out[1:2], w1, "badids seq1")


@pytest.mark.parametrize("scale", [-0.125, 0.0, 2.0e-3])
def test_decode_scale_sign_and_zero(scale):
    """A negative scale is folded into q; a zero scale gives the plain mean of
    V (uniform weights); a tiny scale stays close to it."""
    c = workloads.custom_case("scales", B=3, Hq=14, Hkv=2, D=64, block_size=16,
                              lens=[1, 45, 700], seed=101, scale=scale)
    g = to_gpu(c)
    out = _decode(g, c)
    po, pl = pkv.paged_attention_decode_split(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, c.scale,
                                              64)
    out_s = pkv.split_reduce(po, pl, g.ctx, 64)
    torch.cuda.synchronize()
    want, _ = oracle_decode(c)
    check_fp16(out, want, f"scale {scale}")
    check_fp16(out_s, want, f"split scale {scale}")
