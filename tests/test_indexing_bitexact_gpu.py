"""Bit-exact indexing on every decode path.

The argmax probe: q = 64 e0 and, per sequence, one key row 64 e0 while every
other key row is 0 in dim 0.  At scale 1/8 the logit gap is 512; exp(-512) is
0 in fp32, so each output row is exactly the hot position's V row.  The hot
position sweeps the context (partition and block edges included), so the
probe pins the block-table walk, the partition offsets of the split pass, the
compact grid's item mapping, the fused step's substitution of the new token
from k_new, and the 8-bit cache's head-major addressing.

The block permutation: moving the physical blocks and rewriting the tables
leaves every output bit-identical, because the summation order depends on
logical positions only.

(The GPU indexing pins of the oracle contract; the block tables are the
nanoserve write-up's, "What I built".)"""
import numpy as np
import pytest
import torch

import paged_kv_decode_cache_amd as pkv
import workloads
from gpu_common import DEV, case, needs_gpu, say, to_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]

B, HQ, HKV, D, BS, CTX = 48, 14, 2, 64, 16, 1000
G = HQ // HKV
SCALE = 0.125


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _hot_positions():
    hot = np.linspace(0, CTX - 1, B).astype(int)
    edges = [0, 15, 16, 63, 64, 127, 128, 255, 256, 511, 512, CTX - 2, CTX - 1]
    hot[:len(edges)] = edges
    return hot


def _probe(seed=90, hot=None):
    """The probe case, its modified K pool and q, and the hot positions."""
    c = workloads.custom_case("probe", B=B, Hq=HQ, Hkv=HKV, D=D, block_size=BS,
                              lens=[CTX] * B, seed=seed, scale=SCALE)
    kp = c.k_pool.copy()
    kp[..., 0] = 0.0
    q = np.zeros_like(c.q)
    q[..., 0] = 64.0
    hot = _hot_positions() if hot is None else hot
    for b in range(B):
        t = int(hot[b])
        kp[c.block_tables[b, t // BS], t % BS, :, 0] = 64.0
    return c, kp, q, hot


def _gpu(c, kp, q):
    g = to_gpu(c)
    g.k_pool = _t(kp)
    g.q = _t(q)
    return g


def _expect_rows(got, v_rows, label):
    """got [B, Hq, D] fp16 equals v_rows[b, kv head] bitwise."""
    got = got.cpu().numpy()
    for b in range(B):
        for h in range(HQ):
            want = v_rows[b, h // G]
            assert np.array_equal(got[b, h].view(np.uint16), want.view(np.uint16)), \
                f"{label}: sequence {b}, head {h}"


def _hot_v(c, hot):
    return np.stack([c.v_pool[c.block_tables[b, hot[b] // BS], hot[b] % BS] for b in range(B)])


@pytest.mark.parametrize("P", [64, 256])
@pytest.mark.parametrize("grid", ["direct", "compact"])
def test_split_argmax_probe_bit_exact(P, grid):
    c, kp, q, hot = _probe()
    g = _gpu(c, kp, q)
    say(f"split probe P={P} grid={grid}")
    po, pl = pkv.paged_attention_decode_split(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, SCALE, P,
                                              launch=dict(grid=grid))
    out = pkv.split_reduce(po, pl, g.ctx, P)
    torch.cuda.synchronize()
    v = _hot_v(c, hot)
    _expect_rows(out, v, f"split+merge P={P} {grid}")
    # the hot partition's own row is the V row in fp32, exactly
    po = po.cpu().numpy()
    for b in range(B):
        p = int(hot[b]) // P
        for h in range(HQ):
            assert np.array_equal(po[b, h, p], v[b, h // G].astype(np.float32)), (b, h, p)


@pytest.mark.parametrize("P,launch", [(64, None), (256, None), (256, dict(grid="compact")),
                                      (64, dict(waves=8)), (1024, None)])
def test_step_argmax_probe_bit_exact(P, launch):
    c, kp, q, hot = _probe()
    g = _gpu(c, kp, q)
    say(f"step probe P={P} launch={launch}")
    out = pkv.paged_decode_step(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, SCALE, P, launch=launch)
    torch.cuda.synchronize()
    _expect_rows(out, _hot_v(c, hot), f"step P={P} {launch}")


@pytest.mark.parametrize("P,launch", [(64, None), (256, dict(grid="compact")),
                                      (64, dict(waves=8))])
def test_step_new_token_from_k_new_bit_exact(P, launch):
    """Even sequences' hot key is the step's new token at position ctx-1,
    which the step writes into the pool and must take from k_new/v_new: the
    pool slot holds NaN before the call.  Odd sequences keep their hot key in
    the pool and get a new token with a zero logit."""
    hot = _hot_positions()
    hot[1::2] = np.where(hot[1::2] == CTX - 1, CTX - 3, hot[1::2])  # odd: hot key in the pool
    c, kp, q, hot = _probe(seed=93, hot=hot)
    k_new = c.k_new.copy()
    v_new = c.v_new.copy()
    k_new[..., 0] = 0.0
    vp = c.v_pool.copy()
    for b in range(B):
        slot = int(c.slot_mapping[b])
        kp[slot // BS, slot % BS] = np.nan
        vp[slot // BS, slot % BS] = np.nan
        if b % 2 == 0:
            k_new[b, :, 0] = 64.0
            t = int(hot[b])
            if t != CTX - 1:   # the pool's hot key would win otherwise
                kp[c.block_tables[b, t // BS], t % BS, :, 0] = 0.0
    g = _gpu(c, kp, q)
    g.v_pool = _t(vp)
    g.k_new, g.v_new = _t(k_new), _t(v_new)
    say(f"step new-token probe P={P} launch={launch}")
    out = pkv.paged_decode_step(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, SCALE, P, k_new=g.k_new,
                                v_new=g.v_new, slot_mapping=g.slots, launch=launch)
    torch.cuda.synchronize()
    want = _hot_v(c, hot)
    for b in range(0, B, 2):
        want[b] = v_new[b]
    _expect_rows(out, want, f"step new token P={P} {launch}")
    gk, gv = g.k_pool.cpu().numpy(), g.v_pool.cpu().numpy()
    for b in range(B):
        slot = int(c.slot_mapping[b])
        assert np.array_equal(gk[slot // BS, slot % BS].view(np.uint16), k_new[b].view(np.uint16))
        assert np.array_equal(gv[slot // BS, slot % BS].view(np.uint16), v_new[b].view(np.uint16))


# ---- 8-bit cache -------------------------------------------------------------

def _q8_probe(seed=94):
    """Codes and scales chosen so every product is exact: K scales 1 (hot
    logit 64 * 127 * 1/8 = 1016 above the others), V scales 2^-6 (code *
    scale is an exact fp16 value).  Library layout: codes [NB, Hkv, bs, D],
    scales [NB, Hkv, bs]."""
    c = workloads.custom_case("probe_q8", B=B, Hq=HQ, Hkv=HKV, D=D, block_size=BS,
                              lens=[CTX] * B, seed=seed, scale=SCALE, poison=False)
    rng = np.random.default_rng(seed + 1)
    NB = c.num_blocks
    kc = rng.integers(-127, 128, (NB, BS, HKV, D)).astype(np.int8)
    vc = rng.integers(-127, 128, (NB, BS, HKV, D)).astype(np.int8)
    kc[..., 0] = 0
    hot = _hot_positions()
    for b in range(B):
        t = int(hot[b])
        kc[c.block_tables[b, t // BS], t % BS, :, 0] = 127
    ks = np.ones((NB, BS, HKV), dtype=np.float32)
    vs = np.full((NB, BS, HKV), 2.0 ** -6, dtype=np.float32)
    q = np.zeros_like(c.q)
    q[..., 0] = 64.0
    return c, kc, vc, ks, vs, q, hot


def _q8_gpu(kc, vc, ks, vs):
    return (_t(kc.transpose(0, 2, 1, 3)), _t(vc.transpose(0, 2, 1, 3)), _t(ks.transpose(0, 2, 1)),
            _t(vs.transpose(0, 2, 1)))


def _q8_hot_v(c, vc, hot):
    rows = np.stack([vc[c.block_tables[b, hot[b] // BS], hot[b] % BS] for b in range(B)])
    return (rows.astype(np.float64) * 2.0 ** -6).astype(np.float16)


@pytest.mark.parametrize("path", ["decode", "split64", "split256", "split1024", "step64",
                                  "step256", "step512", "step_compact"])
def test_q8_argmax_probe_bit_exact(path):
    """split1024 is the 8-wave split pass (long partitions, few workgroups);
    step256 and step512 the 8-wave step with the direct merge; step64 the
    4-wave step with the merge through LDS."""
    c, kc, vc, ks, vs, q, hot = _q8_probe()
    g = to_gpu(c)
    g.q = _t(q)
    gq = _q8_gpu(kc, vc, ks, vs)
    say(f"q8 probe {path}")
    if path == "decode":
        out = pkv.paged_attention_decode_q8(g.q, *gq, g.bt, g.ctx, SCALE)
    elif path.startswith("split"):
        P = int(path[5:])
        po, pl = pkv.paged_attention_decode_split_q8(g.q, *gq, g.bt, g.ctx, SCALE, P)
        out = pkv.split_reduce(po, pl, g.ctx, P)
    else:
        P = 256 if path == "step_compact" else int(path[4:])
        out = pkv.paged_decode_step_q8(g.q, *gq, g.bt, g.ctx, SCALE, P)
    torch.cuda.synchronize()
    _expect_rows(out, _q8_hot_v(c, vc, hot), f"q8 {path}")


def test_q8_step_new_token_from_k_new_bit_exact():
    """The 8-bit step quantises the new token in registers and uses it at
    position ctx-1 (the pool row there holds a key that would dominate and a
    zero V row).  k_new = 64 e0 quantises to code 127 with scale 64/127; v_new
    is codes * 2^-6 with a code of +-127, so it quantises back exactly."""
    c, kc, vc, ks, vs, q, hot = _q8_probe(seed=95)
    rng = np.random.default_rng(96)
    k_new = np.zeros((B, HKV, D), dtype=np.float16)
    k_new[..., 0] = 64.0
    codes = rng.integers(-127, 128, (B, HKV, D)).astype(np.int64)
    codes[..., 3] = 127
    v_new = (codes * 2.0 ** -6).astype(np.float16)
    for b in range(B):
        slot = int(c.slot_mapping[b])
        kc[slot // BS, slot % BS, :, 0] = 127      # would win if read from the pool
        vc[slot // BS, slot % BS] = 0
        t = int(hot[b])
        if t != CTX - 1:
            kc[c.block_tables[b, t // BS], t % BS, :, 0] = 0
    g = to_gpu(c)
    g.q = _t(q)
    g.k_new, g.v_new = _t(k_new), _t(v_new)
    gq = _q8_gpu(kc, vc, ks, vs)
    out = pkv.paged_decode_step_q8(g.q, *gq, g.bt, g.ctx, SCALE, 64, k_new=g.k_new,
                                   v_new=g.v_new, slot_mapping=g.slots)
    torch.cuda.synchronize()
    _expect_rows(out, v_new, "q8 step new token")


# ---- block permutation -------------------------------------------------------

def _permuted(c, seed):
    """The case's pools with physical blocks permuted and tables / slots
    rewritten to match."""
    perm = np.random.default_rng(seed).permutation(c.num_blocks)
    kp = np.empty_like(c.k_pool)
    vp = np.empty_like(c.v_pool)
    kp[perm] = c.k_pool
    vp[perm] = c.v_pool
    bt = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    s = c.slot_mapping
    slots = np.where(s >= 0, perm[np.maximum(s, 0) // c.block_size] * c.block_size
                     + np.maximum(s, 0) % c.block_size, -1).astype(np.int64)
    return perm, kp, vp, bt, slots


def _fp16_paths(g, c):
    outs = {}
    for name, P, launch in (("split", 256, None), ("split_compact", 256, dict(grid="compact")),
                            ("split_64", 64, None)):
        po, pl = pkv.paged_attention_decode_split(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, c.scale,
                                                  P, launch=launch)
        outs[name] = pkv.split_reduce(po, pl, g.ctx, P).clone()
    for name, P, launch in (("step", 256, None), ("step_compact", 256, dict(grid="compact")),
                            ("step_8w", 128, dict(waves=8))):
        outs[name] = pkv.paged_decode_step(g.q, g.k_pool.clone(), g.v_pool.clone(), g.bt, g.ctx,
                                           c.scale, P, k_new=g.k_new, v_new=g.v_new,
                                           slot_mapping=g.slots, launch=launch)
    torch.cuda.synchronize()
    return outs


def test_block_permutation_bit_identical_split_and_step():
    c = case("qwen")
    base = _fp16_paths(to_gpu(c), c)
    perm, kp, vp, bt, slots = _permuted(c, 97)
    g = to_gpu(c)
    g.k_pool, g.v_pool, g.bt, g.slots = _t(kp), _t(vp), _t(bt), _t(slots)
    moved = _fp16_paths(g, c)
    for name in base:
        assert torch.equal(base[name].view(torch.int16), moved[name].view(torch.int16)), name


def test_block_permutation_bit_identical_q8():
    c = case("qwen")
    kc, vc, ks, vs = workloads.q8_pools(c)

    def run(g, pools, bt, slots):
        o = {"decode": pkv.paged_attention_decode_q8(g.q, *pools, bt, g.ctx, c.scale)}
        for P in (256, 1024):  # 4- and 8-wave split passes; LDS and direct merges
            po, pl = pkv.paged_attention_decode_split_q8(g.q, *pools, bt, g.ctx, c.scale, P)
            o[f"split{P}"] = pkv.split_reduce(po, pl, g.ctx, P)
            o[f"step{P}"] = pkv.paged_decode_step_q8(g.q, *[x.clone() for x in pools], bt,
                                                     g.ctx, c.scale, P, k_new=g.k_new,
                                                     v_new=g.v_new, slot_mapping=slots)
        torch.cuda.synchronize()
        return o

    g = to_gpu(c)
    base = run(g, _q8_gpu(kc, vc, ks, vs), g.bt, g.slots)
    perm, _, _, bt, slots = _permuted(c, 98)
    pk, pv = np.empty_like(kc), np.empty_like(vc)
    pks, pvs = np.empty_like(ks), np.empty_like(vs)
    pk[perm], pv[perm], pks[perm], pvs[perm] = kc, vc, ks, vs
    moved = run(g, _q8_gpu(pk, pv, pks, pvs), _t(bt), _t(slots))
    for name in base:
        assert torch.equal(base[name].view(torch.int16), moved[name].view(torch.int16)), name
