"""Multi-token append + chunked-prefill attention on the GPU against the fp64
oracle (pools bit-exact after the append, outputs within tolerance)."""
import numpy as np
import pytest
import torch

import paged_kv_decode_cache_amd as pkv
import workloads
from oracle import paged_ref as ref
from gpu_common import DEV, check_fp16, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _prefill(c, kp, vp, max_q=None, q=None, bt=None):
    return pkv.paged_attention_prefill(_t(c.q) if q is None else q, kp, vp,
                                       _t(c.block_tables) if bt is None else bt,
                                       _t(c.context_lens), _t(c.query_start), c.scale,
                                       c.max_q if max_q is None else max_q)


def _append_chunks(c):
    """Pools with the chunk slots poisoned, then the chunks appended on the
    GPU (one slot per chunk token); returns the device pools and the oracle's
    pools after its own append."""
    kp0, vp0 = c.k_pool.copy(), c.v_pool.copy()
    ok = c.chunk_slots >= 0
    blk, off = c.chunk_slots[ok] // c.block_size, c.chunk_slots[ok] % c.block_size
    kp0.view(np.uint16)[blk, off] = workloads.NAN16
    vp0.view(np.uint16)[blk, off] = workloads.NAN16
    kp, vp = _t(kp0), _t(vp0)
    pkv.kv_cache_append(kp, vp, _t(c.k_chunk), _t(c.v_chunk), _t(c.chunk_slots))
    wk, wv = ref.kv_cache_append(kp0, vp0, c.k_chunk, c.v_chunk, c.chunk_slots)
    return kp, vp, wk, wv


CASES = [
    # name, Hq, Hkv, D, bs, ctx, chunk
    ("qwen_chunks", 14, 2, 64, 16, [100, 40, 1000, 17], [100, 8, 512, 1]),
    ("whole_prompts", 14, 2, 64, 16, [64, 33, 300], [64, 33, 300]),
    ("g16_d128_bs32", 16, 1, 128, 32, [70, 600, 5], [70, 33, 5]),
    ("g4_d128", 32, 8, 128, 16, [129, 1024], [16, 200]),
    ("mha_bs64", 4, 4, 64, 64, [200, 64], [37, 64]),
    ("g2_bs256", 4, 2, 64, 256, [513, 1000], [100, 1]),
    ("g12_d64", 12, 1, 64, 16, [90, 600], [33, 100]),
]


@pytest.mark.parametrize("name,Hq,Hkv,D,bs,ctx,chunk", CASES, ids=[x[0] for x in CASES])
def test_append_then_prefill_matches_oracle(name, Hq, Hkv, D, bs, ctx, chunk):
    c = workloads.prefill_case(name, Hq=Hq, Hkv=Hkv, D=D, block_size=bs, ctx=ctx, chunk=chunk,
                               seed=400)
    say(f"prefill {name}: ctx {ctx} chunks {chunk}")
    kp, vp, wk, wv = _append_chunks(c)
    out = _prefill(c, kp, vp)
    torch.cuda.synchronize()
    assert np.array_equal(kp.cpu().numpy().view(np.uint16), wk.view(np.uint16))
    assert np.array_equal(vp.cpu().numpy().view(np.uint16), wv.view(np.uint16))
    want = ref.paged_attention_prefill(c.q, wk, wv, c.block_tables, c.context_lens,
                                       c.query_start, c.scale)
    check_fp16(out, want, f"prefill {name}")


def test_long_chunks_at_context_4096():
    """Four sequences, 512-token chunks ending at position 4095 (q x 4: peaked
    softmax), every row against the oracle."""
    c = workloads.prefill_case("c512", Hq=14, Hkv=2, D=64, block_size=16, ctx=[4096] * 4,
                               chunk=[512] * 4, seed=401, q_mult=4.0)
    say("prefill 4 x 512 rows at ctx 4096")
    out = _prefill(c, _t(c.k_pool), _t(c.v_pool))
    torch.cuda.synchronize()
    want = ref.paged_attention_prefill(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                                       c.query_start, c.scale)
    check_fp16(out, want, "prefill c512")


def test_edge_chunks():
    """Empty chunks, a chunk longer than its context (its first rows precede
    position 0: zeros), a zero-length context, and a max_query_len above the
    longest chunk."""
    c = workloads.prefill_case("edges", Hq=14, Hkv=2, D=64, block_size=16,
                               ctx=[10, 0, 50, 3, 16], chunk=[0, 0, 7, 9, 16], seed=402)
    for max_q in (c.max_q, c.max_q + 40):
        out = _prefill(c, _t(c.k_pool), _t(c.v_pool), max_q=max_q)
        torch.cuda.synchronize()
        want = ref.paged_attention_prefill(c.q, c.k_pool, c.v_pool, c.block_tables,
                                           c.context_lens, c.query_start, c.scale)
        check_fp16(out, want, f"edges max_q={max_q}")
        r = int(c.query_start[3])
        assert int((out[r:r + 6] != 0).sum()) == 0


def test_one_row_chunks_equal_decode():
    c = workloads.custom_case("one_row", B=5, Hq=14, Hkv=2, D=64, block_size=16,
                              lens=[1, 17, 300, 1024, 2000], seed=403)
    qs = np.arange(6, dtype=np.int32)
    out = pkv.paged_attention_prefill(_t(c.q), _t(c.k_pool), _t(c.v_pool), _t(c.block_tables),
                                      _t(c.context_lens), _t(qs), c.scale, 1)
    dec = pkv.paged_attention_decode(_t(c.q), _t(c.k_pool), _t(c.v_pool), _t(c.block_tables),
                                     _t(c.context_lens), c.scale)
    torch.cuda.synchronize()
    want = ref.paged_attention_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                                      c.scale)
    check_fp16(out, want, "one-row prefill")
    assert (out.float() - dec.float()).abs().max().item() <= 2e-3


def test_chunked_prompt_equals_whole_prompt():
    """A 300-token prompt in chunks of 64 (each call with the context written
    so far) gives the rows of one whole-prompt call."""
    c = workloads.prefill_case("whole", Hq=14, Hkv=2, D=64, block_size=16, ctx=[300],
                               chunk=[300], seed=404)
    kp, vp, bt = _t(c.k_pool), _t(c.v_pool), _t(c.block_tables)
    q = _t(c.q)
    whole = pkv.paged_attention_prefill(q, kp, vp, bt, _t(c.context_lens), _t(c.query_start),
                                        c.scale, 300)
    parts = []
    for a in range(0, 300, 64):
        e = min(300, a + 64)
        parts.append(pkv.paged_attention_prefill(
            q[a:e].contiguous(), kp, vp, bt, _t(np.array([e], np.int32)),
            _t(np.array([0, e - a], np.int32)), c.scale, e - a))
    torch.cuda.synchronize()
    got = torch.cat(parts)
    assert (got.float() - whole.float()).abs().max().item() <= 2e-3
    want = ref.paged_attention_prefill(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                                       c.query_start, c.scale)
    check_fp16(got, want, "chunked prompt")


def test_prefill_block_permutation_bit_identical():
    c = workloads.prefill_case("pperm", Hq=14, Hkv=2, D=64, block_size=16, ctx=[500, 77],
                               chunk=[64, 77], seed=405)
    base = _prefill(c, _t(c.k_pool), _t(c.v_pool)).cpu()
    perm = np.random.default_rng(406).permutation(c.num_blocks)
    kp = np.empty_like(c.k_pool)
    vp = np.empty_like(c.v_pool)
    kp[perm] = c.k_pool
    vp[perm] = c.v_pool
    bt = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    moved = _prefill(c, _t(kp), _t(vp), bt=_t(bt)).cpu()
    assert torch.equal(base.view(torch.int16), moved.view(torch.int16))


@pytest.mark.parametrize("scale", [-0.125, 0.0])
def test_prefill_scale_sign_and_zero(scale):
    c = workloads.prefill_case("pscale", Hq=14, Hkv=2, D=64, block_size=16, ctx=[90, 20],
                               chunk=[30, 20], seed=407, scale=scale)
    out = _prefill(c, _t(c.k_pool), _t(c.v_pool))
    torch.cuda.synchronize()
    want = ref.paged_attention_prefill(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                                       c.query_start, c.scale)
    check_fp16(out, want, f"prefill scale {scale}")


# ---- split over context partitions + split_reduce ----------------------------

def _prefill_split(c, kp, vp, P, max_q=None):
    po, pl, rl = pkv.paged_attention_prefill_split(
        _t(c.q), kp, vp, _t(c.block_tables), _t(c.context_lens), _t(c.query_start), c.scale,
        c.max_q if max_q is None else max_q, P)
    return pkv.split_reduce(po, pl, rl, P), po, pl, rl


def _row_lens(c):
    """The length each chunk row carries into the merge: its sequence's
    context length."""
    lens = np.zeros(int(c.query_start[-1]), dtype=np.int32)
    for b in range(len(c.context_lens)):
        lens[c.query_start[b]:c.query_start[b + 1]] = c.context_lens[b]
    return lens


@pytest.mark.parametrize("name,Hq,Hkv,D,bs,ctx,chunk", CASES, ids=[x[0] for x in CASES])
def test_prefill_split_matches_oracle(name, Hq, Hkv, D, bs, ctx, chunk):
    """Split pass + split_reduce against the oracle's prefill, at a partition
    of two blocks (many partitions, rows that see none of the later ones) and
    one of 64 blocks; the per-row lengths exactly the sequences'."""
    c = workloads.prefill_case(name, Hq=Hq, Hkv=Hkv, D=D, block_size=bs, ctx=ctx, chunk=chunk,
                               seed=410)
    want = ref.paged_attention_prefill(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                                       c.query_start, c.scale)
    for P in (2 * bs, 64 * bs):
        say(f"prefill split {name} P={P}")
        out, po, pl, rl = _prefill_split(c, _t(c.k_pool), _t(c.v_pool), P)
        torch.cuda.synchronize()
        check_fp16(out, want, f"prefill split {name} P={P}")
        assert np.array_equal(rl.cpu().numpy(), _row_lens(c))


def test_prefill_split_short_chunks_long_context():
    """The case the split is for: 8 sequences, 64-row chunks ending at
    position 4095 (q x 4: peaked softmax), partitions of 512 and 1024."""
    c = workloads.prefill_case("c64", Hq=14, Hkv=2, D=64, block_size=16, ctx=[4096] * 8,
                               chunk=[64] * 8, seed=411, q_mult=4.0)
    want = ref.paged_attention_prefill(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                                       c.query_start, c.scale)
    for P in (512, 1024):
        say(f"prefill split 8 x 64 rows at ctx 4096, P={P}")
        out, _, _, _ = _prefill_split(c, _t(c.k_pool), _t(c.v_pool), P)
        torch.cuda.synchronize()
        check_fp16(out, want, f"prefill split c64 P={P}")


def test_prefill_split_edge_chunks():
    """As test_edge_chunks, split: rows before position 0 merge to zeros (lse
    -inf in every partition), empty chunks write nothing."""
    c = workloads.prefill_case("edges", Hq=14, Hkv=2, D=64, block_size=16,
                               ctx=[10, 0, 50, 3, 16], chunk=[0, 0, 7, 9, 16], seed=412)
    want = ref.paged_attention_prefill(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                                       c.query_start, c.scale)
    for max_q in (c.max_q, c.max_q + 40):
        for P in (16, 32):
            out, po, pl, rl = _prefill_split(c, _t(c.k_pool), _t(c.v_pool), P, max_q=max_q)
            torch.cuda.synchronize()
            check_fp16(out, want, f"split edges max_q={max_q} P={P}")
            r = int(c.query_start[3])
            assert int((out[r:r + 6] != 0).sum()) == 0
            assert bool(torch.isneginf(pl[r:r + 6, :, :1]).all())
            assert np.array_equal(rl.cpu().numpy(), _row_lens(c))
