"""Pins for the fp64 oracle: each check compares it with something other than
itself (a library routine, a closed form, an invariant, brute force, or the
worked example the pages print).

The ``pin_*`` functions are plain assertions reused by
``test_oracle_mutants.py``, which plants mistakes in the oracle and requires
at least one pin to fail for each.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import paged_ref as ref
from workloads import custom_case, prefill_case, tiny_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _close(a, b, tol=1e-12):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"max abs diff {err:.3e} > {tol * scale:.3e}"


def _paged_from_contiguous(rng, seqs_k, seqs_v, block_size, extra_blocks=3):
    """Scatter per-sequence contiguous K/V [n, Hkv, D] into a paged pool with a
    random block table.  Written independently of the oracle's gather: it
    walks whole blocks, not positions."""
    Hkv, D = seqs_k[0].shape[1:]
    nblk = [-(-k.shape[0] // block_size) for k in seqs_k]
    NB = sum(nblk) + extra_blocks
    kp = np.full((NB, block_size, Hkv, D), np.nan, dtype=np.float16)
    vp = np.full_like(kp, np.nan)
    ids = rng.permutation(NB)
    maxb = max(max(nblk), 1) + 1
    bt = np.full((len(seqs_k), maxb), -1, dtype=np.int32)
    cur = 0
    for s, (K, V) in enumerate(zip(seqs_k, seqs_v)):
        for j in range(nblk[s]):
            blk = ids[cur]
            cur += 1
            bt[s, j] = blk
            rows = K[j * block_size:(j + 1) * block_size]
            kp[blk, :rows.shape[0]] = rows
            vp[blk, :rows.shape[0]] = V[j * block_size:(j + 1) * block_size]
    return kp, vp, bt


def _sdpa_reference(q, seqs_k, seqs_v, scale):
    """torch fp64 scaled_dot_product_attention on contiguous K/V; the GQA
    grouping is made explicit by repeating each KV head over its group."""
    B, Hq, D = q.shape
    Hkv = seqs_k[0].shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        K = torch.from_numpy(seqs_k[b].astype(np.float64)).permute(1, 0, 2)  # [Hkv, n, D]
        V = torch.from_numpy(seqs_v[b].astype(np.float64)).permute(1, 0, 2)
        K = K.repeat_interleave(G, dim=0).unsqueeze(0)                       # [1, Hq, n, D]
        V = V.repeat_interleave(G, dim=0).unsqueeze(0)
        qq = torch.from_numpy(q[b].astype(np.float64)).unsqueeze(0).unsqueeze(2)
        o = torch.nn.functional.scaled_dot_product_attention(qq, K, V, scale=scale)
        out[b] = o[0, :, 0, :].numpy()
    return out


SDPA_SHAPES = [
    # (Hq, Hkv, D, bs, lens)
    (2, 1, 64, 16, [5, 37]),
    (14, 2, 64, 16, [1, 16, 17, 100]),
    (4, 4, 64, 32, [31, 32, 33]),
    (32, 8, 128, 16, [15, 48, 200]),
    (8, 2, 128, 32, [64, 1, 95]),
]


def pin_sdpa(shape_idx: int):
    Hq, Hkv, D, bs, lens = SDPA_SHAPES[shape_idx]
    rng = np.random.default_rng(100 + shape_idx)
    seqs_k = [rng.standard_normal((n, Hkv, D)).astype(np.float16) for n in lens]
    seqs_v = [rng.standard_normal((n, Hkv, D)).astype(np.float16) for n in lens]
    q = rng.standard_normal((len(lens), Hq, D)).astype(np.float16)
    kp, vp, bt = _paged_from_contiguous(rng, seqs_k, seqs_v, bs)
    scale = 1.0 / math.sqrt(D)
    got = ref.paged_attention_decode(q, kp, vp, bt, np.array(lens, np.int32), scale)
    want = _sdpa_reference(q, seqs_k, seqs_v, float(torch.tensor(scale, dtype=torch.float32)))
    _close(got, want, 1e-12)


@pytest.mark.parametrize("shape_idx", range(len(SDPA_SHAPES)))
def test_oracle_matches_torch_sdpa(shape_idx):
    pin_sdpa(shape_idx)


def pin_block_permutation():
    c = custom_case("perm", B=3, Hq=14, Hkv=2, D=64, block_size=16,
                    lens=[17, 100, 64], seed=7)
    lens = c.context_lens
    base = ref.paged_attention_decode(c.q, c.k_pool, c.v_pool, c.block_tables, lens, c.scale)
    rng = np.random.default_rng(8)
    perm = rng.permutation(c.num_blocks)            # old id -> new id
    kp = np.empty_like(c.k_pool)
    vp = np.empty_like(c.v_pool)
    kp[perm] = c.k_pool
    vp[perm] = c.v_pool
    bt = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    moved = ref.paged_attention_decode(c.q, kp, vp, bt, lens, c.scale)
    assert np.array_equal(base, moved)
    assert not np.isnan(base).any()


def test_block_permutation_invariance():
    pin_block_permutation()


def pin_ctx1_is_v_row():
    c = custom_case("ctx1", B=2, Hq=6, Hkv=3, D=64, block_size=16, lens=[1, 1], seed=11)
    out = ref.paged_attention_decode(c.q, c.k_pool, c.v_pool, c.block_tables,
                                     c.context_lens, c.scale)
    for b in range(2):
        blk = c.block_tables[b, 0]
        for h in range(6):
            assert np.array_equal(out[b, h], c.v_pool[blk, 0, h // 2].astype(np.float64))


def test_ctx1_returns_that_v_row():
    pin_ctx1_is_v_row()


def pin_identical_keys_mean_v():
    rng = np.random.default_rng(12)
    n, Hkv, D, Hq = 45, 2, 64, 8
    krow = rng.standard_normal((Hkv, D)).astype(np.float16)
    seqs_k = [np.broadcast_to(krow, (n, Hkv, D)).copy()]
    seqs_v = [rng.standard_normal((n, Hkv, D)).astype(np.float16)]
    kp, vp, bt = _paged_from_contiguous(rng, seqs_k, seqs_v, 16)
    q = rng.standard_normal((1, Hq, D)).astype(np.float16)
    out = ref.paged_attention_decode(q, kp, vp, bt, np.array([n], np.int32), 0.125)
    mean_v = seqs_v[0].astype(np.float64).mean(axis=0)       # [Hkv, D]
    for h in range(Hq):
        _close(out[0, h], mean_v[h // (Hq // Hkv)], 1e-12)
    # q = 0 gives the same mean for arbitrary keys
    seqs_k2 = [rng.standard_normal((n, Hkv, D)).astype(np.float16)]
    kp2, vp2, bt2 = _paged_from_contiguous(rng, seqs_k2, seqs_v, 16)
    out0 = ref.paged_attention_decode(np.zeros_like(q), kp2, vp2, bt2,
                                      np.array([n], np.int32), 0.125)
    for h in range(Hq):
        _close(out0[0, h], mean_v[h // (Hq // Hkv)], 1e-12)


def test_identical_keys_give_mean_of_v():
    pin_identical_keys_mean_v()


def pin_two_token_logistic():
    """n = 2: weights are the logistic function of the logit difference and
    the LSE is logaddexp of the two logits (scipy routines)."""
    rng = np.random.default_rng(13)
    D = 64
    seqs_k = [rng.standard_normal((2, 1, D)).astype(np.float16)]
    seqs_v = [rng.standard_normal((2, 1, D)).astype(np.float16)]
    kp, vp, bt = _paged_from_contiguous(rng, seqs_k, seqs_v, 16)
    q = (rng.standard_normal((1, 1, D)) * 3).astype(np.float16)
    sc = ref.fp32_scale(0.125)
    out, lse = ref.paged_attention_decode(q, kp, vp, bt, np.array([2], np.int32), 0.125,
                                          return_lse=True)
    k = seqs_k[0][:, 0].astype(np.float64)
    v = seqs_v[0][:, 0].astype(np.float64)
    s0 = sc * float(np.dot(k[0], q[0, 0].astype(np.float64)))
    s1 = sc * float(np.dot(k[1], q[0, 0].astype(np.float64)))
    w0 = scipy.special.expit(s0 - s1)
    _close(out[0, 0], w0 * v[0] + (1 - w0) * v[1], 1e-12)
    _close(lse[0, 0], np.logaddexp(s0, s1), 1e-12)


def test_two_token_closed_form():
    pin_two_token_logistic()


SPLIT_SHAPES = [
    # (Hq, Hkv, D, bs, lens, partition sizes)
    (14, 2, 64, 16, [1, 16, 500, 1030], [16, 32, 512, 2048]),
    (4, 1, 128, 32, [33, 700], [32, 64, 1024]),
]


def pin_split_equals_unsplit(idx: int):
    Hq, Hkv, D, bs, lens, psizes = SPLIT_SHAPES[idx]
    c = custom_case("split", B=len(lens), Hq=Hq, Hkv=Hkv, D=D, block_size=bs,
                    lens=lens, seed=20 + idx, q_mult=4.0)
    base, base_lse = ref.paged_attention_decode(c.q, c.k_pool, c.v_pool, c.block_tables,
                                                c.context_lens, c.scale, return_lse=True)
    for P in psizes:
        Pm = -(-c.max_blocks_per_seq * bs // P) + 1        # one spare partition
        po, pl = ref.paged_attention_decode_split(c.q, c.k_pool, c.v_pool, c.block_tables,
                                                  c.context_lens, c.scale, P, Pm)
        out, lse = ref.split_reduce(po, pl, c.context_lens, P)
        _close(out, base, 1e-12)
        _close(lse, base_lse, 1e-12)
        for b, n in enumerate(c.context_lens):
            used = -(-int(n) // P)
            assert np.all(np.isfinite(pl[b, :, :used]))
            assert np.all(np.isneginf(pl[b, :, used:]))


@pytest.mark.parametrize("idx", range(len(SPLIT_SHAPES)))
def test_split_equals_unsplit(idx):
    pin_split_equals_unsplit(idx)


def pin_merge_closed_forms():
    rng = np.random.default_rng(30)
    o = rng.standard_normal((2, 64))
    # an empty partition does not change the other one
    out, L = ref.merge_partitions(np.stack([o[0], np.full(64, np.nan)]), np.array([0.7, -np.inf]))
    _close(out, o[0], 0)
    _close(L, 0.7, 0)
    # two partitions with equal lse: plain average, lse + ln 2
    out, L = ref.merge_partitions(o, np.array([1.5, 1.5]))
    _close(out, o.mean(axis=0), 1e-15)
    _close(L, 1.5 + math.log(2.0), 1e-15)
    # general weights against scipy.special.softmax
    l2 = np.array([0.3, -2.0])
    out, L = ref.merge_partitions(o, l2)
    w = scipy.special.softmax(l2)
    _close(out, w[0] * o[0] + w[1] * o[1], 1e-15)
    _close(L, scipy.special.logsumexp(l2), 1e-15)
    # nothing valid: zeros, -inf
    out, L = ref.merge_partitions(o, np.array([-np.inf, -np.inf]))
    assert np.all(out == 0) and np.isneginf(L)


def test_merge_closed_forms():
    pin_merge_closed_forms()


def pin_gqa_equals_repeated_mha():
    c = custom_case("gqa", B=2, Hq=14, Hkv=2, D=64, block_size=16, lens=[70, 33], seed=40)
    G = 7
    gqa = ref.paged_attention_decode(c.q, c.k_pool, c.v_pool, c.block_tables,
                                     c.context_lens, c.scale)
    kp = np.repeat(c.k_pool, G, axis=2)        # KV head j -> heads jG..jG+G-1
    vp = np.repeat(c.v_pool, G, axis=2)
    mha = ref.paged_attention_decode(c.q, kp, vp, c.block_tables, c.context_lens, c.scale)
    _close(gqa, mha, 1e-12)
    # G = 1 (Hkv = Hq) against per-head single-query calls
    c1 = custom_case("mha", B=1, Hq=3, Hkv=3, D=64, block_size=16, lens=[40], seed=41)
    full = ref.paged_attention_decode(c1.q, c1.k_pool, c1.v_pool, c1.block_tables,
                                      c1.context_lens, c1.scale)
    for h in range(3):
        one = ref.paged_attention_decode(c1.q[:, h:h + 1], c1.k_pool[:, :, h:h + 1],
                                         c1.v_pool[:, :, h:h + 1], c1.block_tables,
                                         c1.context_lens, c1.scale)
        _close(full[:, h], one[:, 0], 1e-12)


def test_gqa_equals_repeated_mha():
    pin_gqa_equals_repeated_mha()


def _brute_force(c):
    """Pure-Python scalar loops with math.exp (tiny inputs only)."""
    B, Hq, D = c.q.shape
    Hkv, bs = c.Hkv, c.block_size
    sc = float(torch.tensor(c.scale, dtype=torch.float32))
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    lse = [[-math.inf] * Hq for _ in range(B)]
    for b in range(B):
        n = int(c.context_lens[b])
        for h in range(Hq):
            kvh = h * Hkv // Hq
            logits = []
            for t in range(n):
                blk = int(c.block_tables[b][t // bs])
                krow = c.k_pool[blk][t % bs][kvh]
                logits.append(sc * sum(float(c.q[b][h][d]) * float(krow[d]) for d in range(D)))
            if not logits:
                continue
            big = max(logits)
            ws = [math.exp(x - big) for x in logits]
            tot = sum(ws)
            lse[b][h] = big + math.log(tot)
            for d in range(D):
                acc = 0.0
                for t in range(n):
                    blk = int(c.block_tables[b][t // bs])
                    acc += ws[t] * float(c.v_pool[blk][t % bs][kvh][d])
                out[b][h][d] = acc / tot
    return np.array(out), np.array(lse)


def pin_brute_force_tiny():
    c = tiny_case()
    got, got_lse = ref.paged_attention_decode(c.q, c.k_pool, c.v_pool, c.block_tables,
                                              c.context_lens, c.scale, return_lse=True)
    want, want_lse = _brute_force(c)
    _close(got, want, 1e-12)
    _close(got_lse, want_lse, 1e-12)
    # also with a GQA group and a ragged tail
    c2 = custom_case("bf", B=2, Hq=4, Hkv=2, D=8, block_size=16, lens=[19, 3], seed=50)
    got2 = ref.paged_attention_decode(c2.q, c2.k_pool, c2.v_pool, c2.block_tables,
                                      c2.context_lens, c2.scale)
    _close(got2, _brute_force(c2)[0], 1e-12)


def test_brute_force_tiny():
    pin_brute_force_tiny()


def pin_ctx0_zero():
    c = custom_case("ctx0", B=2, Hq=2, Hkv=1, D=64, block_size=16, lens=[0, 3], seed=60)
    out, lse = ref.paged_attention_decode(c.q, c.k_pool, c.v_pool, c.block_tables,
                                          c.context_lens, c.scale, return_lse=True)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(out[1]))


def test_ctx0_gives_zeros():
    pin_ctx0_zero()


# ---- cache write ----------------------------------------------------------

def _slots_for_positions(table_row, positions, block_size):
    return np.array([int(table_row[p // block_size]) * block_size + p % block_size
                     for p in positions], dtype=np.int64)


def pin_chunked_prefill_golden():
    """The Day-12 chunked-prefill example: 8-token chunks written into
    4-token blocks occupy 2 blocks after the first pass, 4 after the second."""
    with open(os.path.join(GOLDEN, "chunked_prefill_blocks.json")) as f:
        g = json.load(f)
    bs, chunk = g["block_size"], g["chunk_tokens"]
    passes = len(g["blocks_occupied_after_pass"])
    Hkv, D, NB = 2, 8, 10
    rng = np.random.default_rng(70)
    table = rng.permutation(NB)[: passes * chunk // bs]
    kp = np.full((NB, bs, Hkv, D), np.nan, dtype=np.float16)
    vp = kp.copy()
    for i, want_blocks in enumerate(g["blocks_occupied_after_pass"]):
        pos = list(range(i * chunk, (i + 1) * chunk))
        kn = rng.standard_normal((chunk, Hkv, D)).astype(np.float16)
        vn = rng.standard_normal((chunk, Hkv, D)).astype(np.float16)
        kp, vp = ref.kv_cache_append(kp, vp, kn, vn, _slots_for_positions(table, pos, bs))
        filled = ~np.isnan(kp).any(axis=(2, 3))            # [NB, bs]
        occupied = int(filled.any(axis=1).sum())
        assert occupied == want_blocks
        assert np.all(filled[table[:want_blocks]])          # whole blocks, in table order
        for j, p in enumerate(pos):
            assert np.array_equal(kp[table[p // bs], p % bs], kn[j])
            assert np.array_equal(vp[table[p // bs], p % bs], vn[j])


def test_chunked_prefill_golden():
    pin_chunked_prefill_golden()


def pin_append_brute_force():
    """Element loops: written rows equal the inputs, every other byte of the
    pool is unchanged, and slots naming no row of the pool (negative, or at
    or past num_blocks * block_size) are skipped."""
    rng = np.random.default_rng(71)
    NB, bs, Hkv, D, N = 6, 16, 2, 64, 9
    kp = rng.standard_normal((NB, bs, Hkv, D)).astype(np.float16)
    vp = rng.standard_normal((NB, bs, Hkv, D)).astype(np.float16)
    kn = rng.standard_normal((N, Hkv, D)).astype(np.float16)
    vn = rng.standard_normal((N, Hkv, D)).astype(np.float16)
    slots = rng.choice(NB * bs, size=N, replace=False).astype(np.int64)
    slots[3] = -1
    slots[5] = NB * bs          # one past the last row
    slots[7] = NB * bs + 77
    k2, v2 = ref.kv_cache_append(kp, vp, kn, vn, slots)
    written = {}
    for i, s in enumerate(slots):
        if 0 <= s < NB * bs:
            written[(int(s) // bs, int(s) % bs)] = i
    for blk in range(NB):
        for off in range(bs):
            i = written.get((blk, off))
            srck = kp[blk, off] if i is None else kn[i]
            srcv = vp[blk, off] if i is None else vn[i]
            assert k2[blk, off].tobytes() == srck.tobytes()
            assert v2[blk, off].tobytes() == srcv.tobytes()
    # the inputs are left alone
    assert not np.array_equal(k2, kp)


def test_append_brute_force():
    pin_append_brute_force()


# ---- chunked prefill attention --------------------------------------------

def _chunk_sdpa(q_rows, K, V, ctx, scale, whole):
    """torch fp64 SDPA for one sequence's chunk: q_rows [n, Hq, D] fp16, K/V
    [ctx, Hkv, D] contiguous.  Row i sees keys t <= ctx - n + i: torch's own
    is_causal when the chunk is the whole prompt (n == ctx), otherwise an
    explicit boolean mask.  GQA is made explicit by repeating KV heads."""
    n, Hq, D = q_rows.shape
    G = Hq // K.shape[1]
    Q = torch.from_numpy(q_rows.astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
    Kt = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
    Vt = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
    F = torch.nn.functional
    if whole:
        assert n == ctx
        o = F.scaled_dot_product_attention(Q, Kt.unsqueeze(0), Vt.unsqueeze(0), is_causal=True,
                                           scale=scale)
    else:
        rows = torch.arange(n).unsqueeze(1)
        cols = torch.arange(ctx).unsqueeze(0)
        mask = cols <= rows + (ctx - n)
        o = F.scaled_dot_product_attention(Q, Kt.unsqueeze(0), Vt.unsqueeze(0), attn_mask=mask,
                                           scale=scale)
    return o[0].permute(1, 0, 2).numpy()


PREFILL_SHAPES = [
    # (Hq, Hkv, D, bs, ctx, chunk)
    (2, 1, 64, 16, [37, 5], [37, 5]),               # whole prompts
    (14, 2, 64, 16, [100, 17, 64], [100, 17, 64]),
    (14, 2, 64, 16, [100, 40, 64], [8, 40, 1]),     # chunks after a cached prefix
    (32, 8, 128, 32, [70, 33], [16, 9]),
    (4, 4, 64, 16, [50], [13]),
]


def pin_prefill_sdpa(idx: int):
    Hq, Hkv, D, bs, ctx, chunk = PREFILL_SHAPES[idx]
    rng = np.random.default_rng(300 + idx)
    seqs_k = [rng.standard_normal((n, Hkv, D)).astype(np.float16) for n in ctx]
    seqs_v = [rng.standard_normal((n, Hkv, D)).astype(np.float16) for n in ctx]
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q = rng.standard_normal((int(qs[-1]), Hq, D)).astype(np.float16)
    kp, vp, bt = _paged_from_contiguous(rng, seqs_k, seqs_v, bs)
    scale = 1.0 / math.sqrt(D)
    got = ref.paged_attention_prefill(q, kp, vp, bt, np.array(ctx, np.int32), qs, scale)
    sc = float(torch.tensor(scale, dtype=torch.float32))
    for b in range(len(ctx)):
        want = _chunk_sdpa(q[qs[b]:qs[b + 1]], seqs_k[b], seqs_v[b], ctx[b], sc,
                           whole=chunk[b] == ctx[b])
        _close(got[qs[b]:qs[b + 1]], want, 1e-12)


@pytest.mark.parametrize("idx", range(len(PREFILL_SHAPES)))
def test_prefill_matches_torch_sdpa(idx):
    pin_prefill_sdpa(idx)


def pin_prefill_rows_are_decodes():
    """Row i of a chunk equals a single-token decode of that query over the
    first ctx - n + i + 1 positions (the decode oracle is pinned on its own)."""
    c = prefill_case("rows", Hq=14, Hkv=2, D=64, block_size=16, ctx=[45, 130], chunk=[20, 7],
                     seed=310)
    got = ref.paged_attention_prefill(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                                      c.query_start, c.scale)
    for b in range(c.B):
        n = int(c.chunk_lens[b])
        for i in range(n):
            r = int(c.query_start[b]) + i
            pos = int(c.context_lens[b]) - n + i
            one = ref.paged_attention_decode(c.q[r:r + 1], c.k_pool, c.v_pool,
                                             c.block_tables[b:b + 1],
                                             np.array([pos + 1], np.int32), c.scale)
            _close(got[r], one[0], 1e-12)


def test_prefill_rows_are_decodes():
    pin_prefill_rows_are_decodes()


def pin_prefill_chunking_is_invisible():
    """Chunked prefill is a runtime optimisation only (Inference Engineering,
    Day 12): a prompt processed in chunks -- each call with the context
    written so far -- gives the rows of the whole prompt in one call."""
    c = prefill_case("chunks", Hq=14, Hkv=2, D=64, block_size=16, ctx=[96], chunk=[96],
                     seed=320)
    whole = ref.paged_attention_prefill(c.q, c.k_pool, c.v_pool, c.block_tables,
                                        c.context_lens, c.query_start, c.scale)
    for edges in ([0, 8, 16, 24, 96], [0, 50, 96], [0, 1, 95, 96]):
        for a, e in zip(edges[:-1], edges[1:]):
            part = ref.paged_attention_prefill(c.q[a:e], c.k_pool, c.v_pool, c.block_tables,
                                               np.array([e], np.int32),
                                               np.array([0, e - a], np.int32), c.scale)
            assert np.array_equal(part, whole[a:e])


def test_prefill_chunking_is_invisible():
    pin_prefill_chunking_is_invisible()


def _prefill_brute_force(c):
    """Pure-Python loops with math.exp over the causal prefix of each row."""
    T, Hq, D = c.q.shape
    bs = c.block_size
    sc = float(torch.tensor(c.scale, dtype=torch.float32))
    out = np.zeros((T, Hq, D))
    for b in range(c.B):
        r0, r1 = int(c.query_start[b]), int(c.query_start[b + 1])
        ctx = int(c.context_lens[b])
        for r in range(r0, r1):
            last = ctx - (r1 - r0) + (r - r0)
            for h in range(Hq):
                kvh = h * c.Hkv // Hq
                logits = []
                for t in range(last + 1):
                    blk = int(c.block_tables[b][t // bs])
                    krow = c.k_pool[blk][t % bs][kvh]
                    logits.append(sc * sum(float(c.q[r][h][d]) * float(krow[d])
                                           for d in range(D)))
                if not logits:
                    continue
                big = max(logits)
                ws = [math.exp(x - big) for x in logits]
                tot = sum(ws)
                for d in range(D):
                    acc = 0.0
                    for t in range(last + 1):
                        blk = int(c.block_tables[b][t // bs])
                        acc += ws[t] * float(c.v_pool[blk][t % bs][kvh][d])
                    out[r][h][d] = acc / tot
    return out


def pin_prefill_brute_force():
    c = prefill_case("pbf", Hq=4, Hkv=2, D=8, block_size=16, ctx=[19, 6, 3], chunk=[5, 6, 5],
                     seed=330)
    got = ref.paged_attention_prefill(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                                      c.query_start, c.scale)
    _close(got, _prefill_brute_force(c), 1e-12)
    # the chunk of 5 over a context of 3 has two rows before position 0: zeros
    r0 = int(c.query_start[2])
    assert np.all(got[r0:r0 + 2] == 0)


def test_prefill_brute_force():
    pin_prefill_brute_force()


def pin_prefill_block_permutation():
    c = prefill_case("pperm", Hq=14, Hkv=2, D=64, block_size=16, ctx=[77, 30], chunk=[12, 30],
                     seed=340)
    base = ref.paged_attention_prefill(c.q, c.k_pool, c.v_pool, c.block_tables,
                                       c.context_lens, c.query_start, c.scale)
    perm = np.random.default_rng(341).permutation(c.num_blocks)
    kp = np.empty_like(c.k_pool)
    vp = np.empty_like(c.v_pool)
    kp[perm] = c.k_pool
    vp[perm] = c.v_pool
    bt = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    moved = ref.paged_attention_prefill(c.q, kp, vp, bt, c.context_lens, c.query_start, c.scale)
    assert np.array_equal(base, moved)
    assert not np.isnan(base).any()


def test_prefill_block_permutation():
    pin_prefill_block_permutation()


# ---- 8-bit cache --------------------------------------------------------------

def _f32(v):
    """Round a Python float to the nearest fp32 value."""
    import struct
    return struct.unpack("f", struct.pack("f", v))[0]


def _quantize_brute(row):
    """Per-row int8 quantisation with scalar Python arithmetic, each step
    rounded to fp32 as the format prescribes (an fp32 op computed in fp64 and
    rounded once is the correctly rounded fp32 result for *, /)."""
    xs = [float(v) for v in row]
    amax = max(abs(v) for v in xs)
    if amax == 0:
        return [0] * len(xs), 0.0
    inv = _f32(127.0 / amax)
    codes = [max(-127, min(127, round(_f32(v * inv)))) for v in xs]   # round(): half to even
    return codes, _f32(amax / 127.0)


def pin_q8_brute_force():
    rng = np.random.default_rng(600)
    rows = [rng.standard_normal(64).astype(np.float16) for _ in range(6)]
    rows.append(np.zeros(64, np.float16))
    tie = np.zeros(64, np.float16)
    tie[0], tie[1], tie[2], tie[3] = 127.0, 63.5, -0.5, 1.5      # inv = 1: ties at .5
    rows.append(tie)
    rows.append((rng.standard_normal(128) * 1e-3).astype(np.float16))
    for r in rows:
        codes, scale = ref.quantize_rows_q8(r[None])
        want_c, want_s = _quantize_brute(r)
        assert list(codes[0]) == want_c
        assert float(scale[0]) == want_s
    c, _ = ref.quantize_rows_q8(tie[None])
    assert list(c[0, :4]) == [127, 64, 0, 2]


def test_q8_brute_force():
    pin_q8_brute_force()


def pin_q8_roundtrip_bound():
    """Each value comes back within half a quantisation step; the largest
    magnitude of a row maps to +-127."""
    rng = np.random.default_rng(601)
    x = (rng.standard_normal((200, 64)) * rng.uniform(0.01, 8, (200, 1))).astype(np.float16)
    codes, scales = ref.quantize_rows_q8(x)
    back = ref.dequantize_pool_q8(codes[None], scales[None])[0]
    err = np.abs(back - x.astype(np.float64))
    assert np.all(err <= scales[:, None].astype(np.float64) * (0.5 + 1e-6))
    assert np.all(np.abs(codes) <= 127)
    top = np.argmax(np.abs(x.astype(np.float32)), axis=1)
    assert np.all(np.abs(codes[np.arange(200), top]) == 127)


def test_q8_roundtrip_bound():
    pin_q8_roundtrip_bound()


def pin_q8_exact_rows_match_fp16_attention():
    """K/V rows that are integer multiples c * 2^-k with max |c| = 127
    quantise exactly, so attention over the 8-bit cache equals the fp16
    oracle over the same values."""
    c = custom_case("q8exact", B=3, Hq=14, Hkv=2, D=64, block_size=16, lens=[20, 100, 7],
                    seed=602, poison=False)
    rng = np.random.default_rng(603)
    shape = c.k_pool.shape
    def exact_pool():
        ints = rng.integers(-127, 128, shape)
        ints[..., 0] = 127                                     # every row reaches 127
        k = rng.integers(4, 9, shape[:3])[..., None]           # per-row power-of-two step
        return (ints * np.exp2(-k.astype(np.float64))).astype(np.float16)
    kp, vp = exact_pool(), exact_pool()
    kq, ks = ref.quantize_rows_q8(kp)
    vq, vs = ref.quantize_rows_q8(vp)
    assert np.array_equal(ref.dequantize_pool_q8(kq, ks), kp.astype(np.float64))
    got = ref.paged_attention_decode(c.q, ref.dequantize_pool_q8(kq, ks),
                                     ref.dequantize_pool_q8(vq, vs), c.block_tables,
                                     c.context_lens, c.scale)
    want = ref.paged_attention_decode(c.q, kp, vp, c.block_tables, c.context_lens, c.scale)
    assert np.array_equal(got, want)


def test_q8_exact_rows_match_fp16_attention():
    pin_q8_exact_rows_match_fp16_attention()


def pin_q8_append_brute_force():
    rng = np.random.default_rng(604)
    NB, bs, Hkv, D = 6, 16, 2, 64
    kc = rng.integers(-127, 128, (NB, bs, Hkv, D)).astype(np.int8)
    vc = rng.integers(-127, 128, (NB, bs, Hkv, D)).astype(np.int8)
    ks = rng.uniform(0, 1, (NB, bs, Hkv)).astype(np.float32)
    vs = rng.uniform(0, 1, (NB, bs, Hkv)).astype(np.float32)
    kn = rng.standard_normal((5, Hkv, D)).astype(np.float16)
    vn = rng.standard_normal((5, Hkv, D)).astype(np.float16)
    slots = np.array([3, -1, 40, 95, NB * bs], np.int64)
    gk, gv, gks, gvs = ref.kv_cache_append_q8(kc, vc, ks, vs, kn, vn, slots)
    wk, wv, wks, wvs = kc.copy(), vc.copy(), ks.copy(), vs.copy()
    for i, sl in enumerate(slots):
        if sl < 0 or sl >= NB * bs:
            continue
        for h in range(Hkv):
            ck, sk = _quantize_brute(kn[i, h])
            cv, sv = _quantize_brute(vn[i, h])
            for d in range(D):
                wk[sl // bs, sl % bs, h, d] = ck[d]
                wv[sl // bs, sl % bs, h, d] = cv[d]
            wks[sl // bs, sl % bs, h] = sk
            wvs[sl // bs, sl % bs, h] = sv
    for g, w in ((gk, wk), (gv, wv), (gks, wks), (gvs, wvs)):
        assert np.array_equal(g, w)


def test_q8_append_brute_force():
    pin_q8_append_brute_force()


ALL_PINS = (
    [lambda i=i: pin_sdpa(i) for i in range(len(SDPA_SHAPES))]
    + [pin_block_permutation, pin_ctx1_is_v_row, pin_identical_keys_mean_v,
       pin_two_token_logistic, pin_merge_closed_forms, pin_gqa_equals_repeated_mha,
       pin_brute_force_tiny, pin_ctx0_zero, pin_chunked_prefill_golden,
       pin_append_brute_force, pin_prefill_rows_are_decodes,
       pin_prefill_chunking_is_invisible, pin_prefill_brute_force,
       pin_prefill_block_permutation, pin_q8_brute_force, pin_q8_roundtrip_bound,
       pin_q8_exact_rows_match_fp16_attention, pin_q8_append_brute_force]
    + [lambda i=i: pin_prefill_sdpa(i) for i in range(len(PREFILL_SHAPES))]
    + [lambda i=i: pin_split_equals_unsplit(i) for i in range(len(SPLIT_SHAPES))]
)
