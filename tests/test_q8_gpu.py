"""8-bit KV cache on the GPU: the quantising cache write bit-exact against the
oracle's, and decode (unsplit, split + merge) over int8 codes against the
fp64 oracle on the dequantised cache."""
import numpy as np
import pytest
import torch

import paged_kv_decode_cache_amd as pkv
import workloads
from oracle import paged_ref as ref
from gpu_common import DEV, PARTIAL_ATOL, case, check_fp16, host64, needs_gpu, say, to_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _lib_codes(c):
    """Codes [NB, bs, Hkv, D] (the oracle's order) in the library's
    head-major layout [NB, Hkv, bs, D]."""
    return c.transpose(0, 2, 1, 3)


def _oracle_codes(g):
    """Device codes [NB, Hkv, bs, D] back in the oracle's order."""
    return g.cpu().numpy().transpose(0, 2, 1, 3)


def _gpu_q8(kc, vc, ks, vs):
    """Device copies in the library's layout (codes [NB, Hkv, bs, D], scales
    [NB, Hkv, bs])."""
    return (_t(_lib_codes(kc)), _t(_lib_codes(vc)), _t(ks.transpose(0, 2, 1)),
            _t(vs.transpose(0, 2, 1)))


def _oracle_decode_q8(c, kc, vc, ks, vs, seqs=None, q=None, ctx=None):
    kd = ref.dequantize_pool_q8(kc, ks)
    vd = ref.dequantize_pool_q8(vc, vs)
    return ref.paged_attention_decode(c.q if q is None else q, kd, vd, c.block_tables,
                                      c.context_lens if ctx is None else ctx, c.scale,
                                      return_lse=True, seqs=seqs)


APPEND_SHAPES = [(2, 64, 16), (8, 128, 32), (1, 64, 256), (4, 128, 16)]


@pytest.mark.parametrize("Hkv,D,bs", APPEND_SHAPES)
def test_append_q8_bit_exact(Hkv, D, bs):
    rng = np.random.default_rng(700 + D + bs)
    NB, N = 12, 40
    kc = rng.integers(-127, 128, (NB, bs, Hkv, D), dtype=np.int8)
    vc = rng.integers(-127, 128, (NB, bs, Hkv, D), dtype=np.int8)
    ks = rng.uniform(0, 1, (NB, bs, Hkv)).astype(np.float32)
    vs = rng.uniform(0, 1, (NB, bs, Hkv)).astype(np.float32)
    kn = (rng.standard_normal((N, Hkv, D)) * rng.uniform(1e-3, 8, (N, Hkv, 1))).astype(np.float16)
    vn = (rng.standard_normal((N, Hkv, D)) * rng.uniform(1e-3, 8, (N, Hkv, 1))).astype(np.float16)
    kn[0] = 0.0                                   # zero rows: codes 0, scale 0
    kn[1, :, :4] = np.array([127.0, 63.5, -0.5, 1.5], np.float16)   # inv = 1: ties
    kn[1, :, 4:] = 0.0
    slots = rng.permutation(NB * bs)[:N].astype(np.int64)
    slots[5], slots[9] = -1, NB * bs + 3          # skipped
    g = list(_gpu_q8(kc, vc, ks, vs))
    pkv.kv_cache_append_q8(*g, _t(kn), _t(vn), _t(slots))
    torch.cuda.synchronize()
    wk, wv, wks, wvs = ref.kv_cache_append_q8(kc, vc, ks, vs, kn, vn, slots)
    assert np.array_equal(_oracle_codes(g[0]), wk)
    assert np.array_equal(_oracle_codes(g[1]), wv)
    assert np.array_equal(g[2].cpu().numpy().transpose(0, 2, 1).view(np.uint32), wks.view(np.uint32))
    assert np.array_equal(g[3].cpu().numpy().transpose(0, 2, 1).view(np.uint32), wvs.view(np.uint32))


Q8_CASES = ["tiny", "qwen", "sweep:32:4096", "sweep:1:128", "sweep:8:2048", "long:1:32768"]


@pytest.mark.parametrize("name", Q8_CASES)
def test_decode_q8_matches_oracle(name):
    c = case(name)
    say(f"decode q8 {name}")
    kc, vc, ks, vs = workloads.q8_pools(c)
    g = to_gpu(c)
    out = pkv.paged_attention_decode_q8(g.q, *_gpu_q8(kc, vc, ks, vs), g.bt, g.ctx, c.scale)
    torch.cuda.synchronize()
    want, _ = _oracle_decode_q8(c, kc, vc, ks, vs)
    check_fp16(out, want, f"decode q8 {name}")


@pytest.mark.parametrize("name,P", [("qwen", 256), ("sweep:32:4096", 512), ("tiny", 16),
                                    ("long:1:32768", 512), ("sweep:8:1024", 64),
                                    # 8-wave split passes (long partitions, <= 256 workgroups)
                                    ("sweep:32:4096", 1024), ("long:4:32768", 1024),
                                    ("sweep:8:4096", 2048)])
def test_split_q8_matches_oracle(name, P):
    c = case(name)
    say(f"split q8 {name} P={P}")
    kc, vc, ks, vs = workloads.q8_pools(c)
    g = to_gpu(c)
    Pm = c.max_partitions(P)
    po, pl = pkv.paged_attention_decode_split_q8(g.q, *_gpu_q8(kc, vc, ks, vs), g.bt, g.ctx,
                                                 c.scale, P, Pm)
    out, lse = pkv.split_reduce(po, pl, g.ctx, P, want_lse=True)
    torch.cuda.synchronize()
    want, want_lse = _oracle_decode_q8(c, kc, vc, ks, vs)
    check_fp16(out, want, f"split q8 {name}")
    fin = np.isfinite(want_lse)
    assert float(np.abs(host64(lse)[fin] - want_lse[fin]).max()) <= PARTIAL_ATOL
    wpo, wpl = ref.paged_attention_decode_split(c.q, ref.dequantize_pool_q8(kc, ks),
                                                ref.dequantize_pool_q8(vc, vs), c.block_tables,
                                                c.context_lens, c.scale, P, Pm)
    valid = np.isfinite(wpl)
    assert np.array_equal(np.isneginf(host64(pl)), np.isneginf(wpl))
    assert float(np.abs(host64(po)[valid] - wpo[valid]).max()) <= PARTIAL_ATOL


@pytest.mark.parametrize("Hq,Hkv,D,bs,lens", [
    (16, 1, 128, 32, [40, 700, 1]),
    (32, 8, 128, 16, [100, 1, 900]),
    (4, 4, 64, 64, [3, 77, 500]),
    (14, 2, 64, 16, [0, 1, 15, 16, 17, 1000]),
    (12, 1, 64, 16, [1, 90, 700]),
])
def test_decode_q8_edge_shapes(Hq, Hkv, D, bs, lens):
    c = workloads.custom_case("q8edge", B=len(lens), Hq=Hq, Hkv=Hkv, D=D, block_size=bs,
                              lens=lens, seed=710)
    kc, vc, ks, vs = workloads.q8_pools(c)
    g = to_gpu(c)
    gq = _gpu_q8(kc, vc, ks, vs)
    out = pkv.paged_attention_decode_q8(g.q, *gq, g.bt, g.ctx, c.scale)
    po, pl = pkv.paged_attention_decode_split_q8(g.q, *gq, g.bt, g.ctx, c.scale, 64)
    out_s = pkv.split_reduce(po, pl, g.ctx, 64)
    torch.cuda.synchronize()
    want, _ = _oracle_decode_q8(c, kc, vc, ks, vs)
    check_fp16(out, want, f"q8 edge {Hq}/{Hkv}/{D}/{bs}")
    check_fp16(out_s, want, f"q8 edge split {Hq}/{Hkv}/{D}/{bs}")


def test_q8_lognormal_lengths_d128():
    """The skewed configuration's head shape (Hq=32, Hkv=8, D=128) with 32
    lognormal lengths (median 1024, clipped to [16, 8192])."""
    rng = np.random.default_rng(720)
    lens = np.clip(workloads.skewed_lengths(rng, B=32), 16, 8192)
    c = workloads.custom_case("q8lognormal", B=32, Hq=32, Hkv=8, D=128, block_size=16,
                              lens=lens, seed=721)
    kc, vc, ks, vs = workloads.q8_pools(c)
    g = to_gpu(c)
    gq = _gpu_q8(kc, vc, ks, vs)
    out = pkv.paged_attention_decode_q8(g.q, *gq, g.bt, g.ctx, c.scale)
    po, pl = pkv.paged_attention_decode_split_q8(g.q, *gq, g.bt, g.ctx, c.scale, 512)
    out_s = pkv.split_reduce(po, pl, g.ctx, 512)
    torch.cuda.synchronize()
    want, _ = _oracle_decode_q8(c, kc, vc, ks, vs)
    check_fp16(out, want, "q8 lognormal")
    check_fp16(out_s, want, "q8 lognormal split")


def test_q8_step_append_then_decode():
    """One decode step on the 8-bit cache: quantising append of each
    sequence's new token at position ctx-1, then decode, against the oracle's
    append and decode."""
    c = case("qwen")
    kc, vc, ks, vs = workloads.q8_pools(c)
    g = to_gpu(c)
    gq = _gpu_q8(kc, vc, ks, vs)
    pkv.kv_cache_append_q8(*gq, g.k_new, g.v_new, g.slots)
    out = pkv.paged_attention_decode_q8(g.q, *gq, g.bt, g.ctx, c.scale)
    torch.cuda.synchronize()
    wk, wv, wks, wvs = ref.kv_cache_append_q8(kc, vc, ks, vs, c.k_new, c.v_new, c.slot_mapping)
    assert np.array_equal(_oracle_codes(gq[0]), wk)
    assert np.array_equal(_oracle_codes(gq[1]), wv)
    want, _ = _oracle_decode_q8(c, wk, wv, wks, wvs)
    check_fp16(out, want, "q8 step")


def test_q8_quantisation_error_against_fp16():
    """The format's own error (not the kernel's): the qwen cache quantised on
    the GPU, position by position, then decoded, against the fp16 oracle on
    the original cache.  N(0,1) data: the bound is loose (0.05) and the
    measured error is reported."""
    c = case("qwen")
    NB, bs, Hkv, D = c.k_pool.shape
    rows = np.nonzero(~np.isnan(c.k_pool[..., 0, 0].astype(np.float32)).ravel())[0]
    slots = rows.astype(np.int64)
    kn = c.k_pool.reshape(NB * bs, Hkv, D)[rows]
    vn = c.v_pool.reshape(NB * bs, Hkv, D)[rows]
    gq = (torch.zeros((NB, Hkv, bs, D), dtype=torch.int8, device=DEV),
          torch.zeros((NB, Hkv, bs, D), dtype=torch.int8, device=DEV),
          torch.zeros((NB, Hkv, bs), dtype=torch.float32, device=DEV),
          torch.zeros((NB, Hkv, bs), dtype=torch.float32, device=DEV))
    pkv.kv_cache_append_q8(*gq, _t(kn), _t(vn), _t(slots))
    g = to_gpu(c)
    out = pkv.paged_attention_decode_q8(g.q, *gq, g.bt, g.ctx, c.scale)
    torch.cuda.synchronize()
    want16 = ref.paged_attention_decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                                        c.scale)
    err = float(np.abs(host64(out) - want16).max())
    say(f"8-bit cache vs fp16 cache, qwen: max abs difference {err:.4f}")
    assert err <= 0.05


# ---- fused decode step over the 8-bit cache ---------------------------------

def _step_q8(g, gq, c, P, ws=None, slots=None, want_lse=True):
    return pkv.paged_decode_step_q8(g.q, *gq, g.bt, g.ctx, c.scale, P, k_new=g.k_new,
                                    v_new=g.v_new, slot_mapping=g.slots if slots is None else slots,
                                    workspace=ws, want_lse=want_lse)


def _check_pools_q8(gq, want):
    """The device 8-bit cache equals the oracle's, bitwise (codes and scales,
    NaN scales of unattended rows included)."""
    wk, wv, wks, wvs = want
    assert np.array_equal(_oracle_codes(gq[0]), wk)
    assert np.array_equal(_oracle_codes(gq[1]), wv)
    assert np.array_equal(gq[2].cpu().numpy().transpose(0, 2, 1).view(np.uint32),
                          wks.view(np.uint32))
    assert np.array_equal(gq[3].cpu().numpy().transpose(0, 2, 1).view(np.uint32),
                          wvs.view(np.uint32))


def _check_workspace_restored(ws):
    assert int(ws.counters.abs().sum()) == 0
    assert bool((ws.partial_out.view(torch.int32) == 0).all())
    assert bool((ws.partial_lse.view(torch.int32) == 0).all())


@pytest.mark.parametrize("name,P", [("tiny", 16), ("qwen", 256), ("qwen", 1024),
                                    ("sweep:32:4096", 1024), ("sweep:8:2048", 256),
                                    ("long:1:32768", 1024), ("long:1:32768", 512),
                                    ("long:4:32768", 512)])
def test_q8_step_matches_append_then_decode(name, P):
    """The fused 8-bit step (quantising append + split pass + merge in one
    launch) against the oracle's kv_cache_append_q8 followed by its decode
    over the dequantised cache; the cache write bit-exact."""
    c = case(name)
    say(f"q8 step {name} P={P}")
    kc, vc, ks, vs = workloads.q8_pools(c)
    g = to_gpu(c)
    gq = _gpu_q8(kc, vc, ks, vs)
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    out, lse = _step_q8(g, gq, c, P, ws)
    torch.cuda.synchronize()
    want_pools = ref.kv_cache_append_q8(kc, vc, ks, vs, c.k_new, c.v_new, c.slot_mapping)
    _check_pools_q8(gq, want_pools)
    want, want_lse = _oracle_decode_q8(c, *want_pools)
    check_fp16(out, want, f"q8 step {name}")
    g_lse = host64(lse)
    assert np.array_equal(np.isneginf(g_lse), np.isneginf(want_lse))
    fin = np.isfinite(want_lse)
    assert float(np.abs(g_lse[fin] - want_lse[fin]).max()) <= PARTIAL_ATOL
    _check_workspace_restored(ws)


def test_q8_step_equals_three_launch_path_and_repeats():
    """Two steps in a row on one workspace: each equals the three-launch
    8-bit step (append + split pass + split_reduce) on its own copy of the
    cache, and every call leaves the workspace ready for the next."""
    c = case("qwen")
    P = 256
    kc, vc, ks, vs = workloads.q8_pools(c)
    g = to_gpu(c)
    gq = _gpu_q8(kc, vc, ks, vs)
    gq3 = _gpu_q8(kc, vc, ks, vs)
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    for rep in range(2):
        out = _step_q8(g, gq, c, P, ws, want_lse=False)
        pkv.kv_cache_append_q8(*gq3, g.k_new, g.v_new, g.slots)
        po, pl = pkv.paged_attention_decode_split_q8(g.q, *gq3, g.bt, g.ctx, c.scale, P)
        out3 = pkv.split_reduce(po, pl, g.ctx, P)
        torch.cuda.synchronize()
        for a_, b_ in zip(gq, gq3):
            assert torch.equal(a_.view(torch.uint8), b_.view(torch.uint8)), f"cache rep {rep}"
        err = float((out.float() - out3.float()).abs().max())
        assert err <= 2e-3, f"rep {rep}: {err}"
        _check_workspace_restored(ws)


def test_q8_step_edge_lengths_and_slots():
    """Context lengths 0, 1, a block, a block + 1 and several partitions; a
    skipped slot (-1) writes nothing and attends over the cache as it is."""
    c = workloads.custom_case("q8_step_edges", B=6, Hq=14, Hkv=2, D=64, block_size=16,
                              lens=[0, 1, 16, 17, 511, 1300], seed=120, q_mult=4.0)
    kc, vc, ks, vs = workloads.q8_pools(c)
    # the skipped sequence's position ctx-1 keeps the pool's own (finite) row
    slots = c.slot_mapping.copy()
    skip = 4
    blk = c.block_tables[skip, (c.context_lens[skip] - 1) // c.block_size]
    off = (c.context_lens[skip] - 1) % c.block_size
    ks[blk, off] = 0.02
    vs[blk, off] = 0.03
    slots[skip] = -1
    for P in (16, 512, 2048):
        g = to_gpu(c)
        gq = _gpu_q8(kc, vc, ks, vs)
        s_gpu = torch.from_numpy(slots).to(g.q.device)
        out, lse = _step_q8(g, gq, c, P, slots=s_gpu)
        torch.cuda.synchronize()
        want_pools = ref.kv_cache_append_q8(kc, vc, ks, vs, c.k_new, c.v_new, slots)
        _check_pools_q8(gq, want_pools)
        want, _ = _oracle_decode_q8(c, *want_pools)
        check_fp16(out, want, f"q8 step edges P={P}")
        assert int((out[0] != 0).sum()) == 0


@pytest.mark.parametrize("P", [256, 1024])
@pytest.mark.parametrize("Hq,Hkv,D,bs", [(16, 1, 128, 32), (32, 8, 128, 16), (12, 1, 64, 16)])
def test_q8_step_other_shapes(Hq, Hkv, D, bs, P):
    """Other shapes at 10 and at 3 partitions per pair."""
    c = workloads.custom_case("q8_step_shapes", B=4, Hq=Hq, Hkv=Hkv, D=D, block_size=bs,
                              lens=[3, 200, 1000, 2500], seed=121)
    kc, vc, ks, vs = workloads.q8_pools(c)
    g = to_gpu(c)
    gq = _gpu_q8(kc, vc, ks, vs)
    out = _step_q8(g, gq, c, P, want_lse=False)
    torch.cuda.synchronize()
    want_pools = ref.kv_cache_append_q8(kc, vc, ks, vs, c.k_new, c.v_new, c.slot_mapping)
    _check_pools_q8(gq, want_pools)
    want, _ = _oracle_decode_q8(c, *want_pools)
    check_fp16(out, want, f"q8 step shapes {Hq}/{Hkv}/{D}/{bs}")


@pytest.mark.parametrize("P", [256, 64])
def test_q8_step_in_hip_graph_replays(P):
    """Replays of a captured 8-bit step, with eager work and synchronisation
    between them, equal the eager result bitwise (the append rewrites the same
    slots with the same codes, so every replay sees the same cache); at 4
    and at 16 partitions per pair."""
    c = case("sweep:32:1024")
    kc, vc, ks, vs = workloads.q8_pools(c)
    g = to_gpu(c)
    gq = _gpu_q8(kc, vc, ks, vs)
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    out = torch.empty((c.B, c.Hq, c.D), dtype=torch.float16, device=g.q.device)
    eager = _step_q8(g, gq, c, P, ws, want_lse=False).clone()
    torch.cuda.synchronize()

    def launch():
        pkv.paged_decode_step_q8(g.q, *gq, g.bt, g.ctx, c.scale, P, k_new=g.k_new,
                                 v_new=g.v_new, slot_mapping=g.slots, workspace=ws, out=out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch()
    for rep in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        _check_workspace_restored(ws)
        junk = torch.randn(1024, device=g.q.device).sum()
        torch.cuda.synchronize()
        del junk


def test_q8_step_ragged_many_partitions():
    """A ragged batch at a small partition (up to 128 partitions per sequence,
    most of the grid's workgroups empty): the merge walks many batches of
    rows.  Every sequence against the oracle's 8-bit append + decode; the
    cache write checked whole."""
    rng = np.random.default_rng(140)
    lens = rng.integers(1, 8193, 24).tolist()
    lens[0], lens[1] = 8192, 1
    c = workloads.custom_case("q8_ragged", B=24, Hq=14, Hkv=2, D=64, block_size=16, lens=lens,
                              seed=141)
    kc, vc, ks, vs = workloads.q8_pools(c)
    g = to_gpu(c)
    gq = _gpu_q8(kc, vc, ks, vs)
    P = 64
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    out = _step_q8(g, gq, c, P, ws, want_lse=False)
    torch.cuda.synchronize()
    want_pools = ref.kv_cache_append_q8(kc, vc, ks, vs, c.k_new, c.v_new, c.slot_mapping)
    _check_pools_q8(gq, want_pools)
    want, _ = _oracle_decode_q8(c, *want_pools)
    check_fp16(out, want, "q8 step ragged")
    _check_workspace_restored(ws)


def test_q8_step_wide_merge_large_group():
    """The 8-bit step with groups of 16 query heads at long contexts with few
    workgroups, where it takes 8 waves for the merge: against the oracle's
    8-bit append + decode; the cache write bit-exact."""
    c = workloads.custom_case("q8_step_wide_g16", B=2, Hq=32, Hkv=2, D=64, block_size=16,
                              lens=[16384, 9001], seed=151)
    kc, vc, ks, vs = workloads.q8_pools(c)
    g = to_gpu(c)
    gq = _gpu_q8(kc, vc, ks, vs)
    P = 1024
    say(f"q8 step wide merge G=16 P={P}")
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    out, lse = _step_q8(g, gq, c, P, ws)
    torch.cuda.synchronize()
    want_pools = ref.kv_cache_append_q8(kc, vc, ks, vs, c.k_new, c.v_new, c.slot_mapping)
    _check_pools_q8(gq, want_pools)
    want, want_lse = _oracle_decode_q8(c, *want_pools)
    check_fp16(out, want, "q8 step wide merge G=16")
    g_lse = host64(lse)
    fin = np.isfinite(want_lse)
    assert float(np.abs(g_lse[fin] - want_lse[fin]).max()) <= PARTIAL_ATOL



def test_q8_step_two_level_merge_g16_d128():
    """The 8-bit step's two-level merge with groups of 16 heads at head_dim
    128 (partition counts 17..200 at P=32), against the oracle's 8-bit append
    + decode; the cache write bit-exact and the workspace zero afterwards."""
    rng = np.random.default_rng(180)
    P = 32
    nps = [1, 17, 33, 64, 129, 200]
    lens = [max(1, n * P - int(rng.integers(0, P))) for n in nps]
    c = workloads.custom_case("q8_step_two_level_g16", B=len(lens), Hq=32, Hkv=2, D=128,
                              block_size=16, lens=lens, seed=181)
    kc, vc, ks, vs = workloads.q8_pools(c)
    g = to_gpu(c)
    gq = _gpu_q8(kc, vc, ks, vs)
    say(f"q8 step two-level G=16 D=128 P={P} partitions={nps}")
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    out, lse = _step_q8(g, gq, c, P, ws)
    torch.cuda.synchronize()
    want_pools = ref.kv_cache_append_q8(kc, vc, ks, vs, c.k_new, c.v_new, c.slot_mapping)
    _check_pools_q8(gq, want_pools)
    want, want_lse = _oracle_decode_q8(c, *want_pools)
    check_fp16(out, want, "q8 step two-level G=16 D=128")
    g_lse = host64(lse)
    fin = np.isfinite(want_lse)
    assert float(np.abs(g_lse[fin] - want_lse[fin]).max()) <= PARTIAL_ATOL
    _check_workspace_restored(ws)


@pytest.mark.parametrize("P", [256, 1024])
def test_q8_step_8wave_stress_against_three_launch_path(P):
    """20 fused 8-bit steps with new queries and new context lengths, each
    against the 8-bit split pass + split_reduce at the same partition size:
    at P=256 four partitions per pair (the 8-wave direct merge), at P=1024
    one (the 8-wave split pass beside it).  Each step is also repeated on
    the same inputs and must match itself bitwise."""
    c = case("sweep:32:1024")
    assert c.max_partitions(256) == 4
    kc, vc, ks, vs = workloads.q8_pools(c)
    g = to_gpu(c)
    gq = _gpu_q8(kc, vc, ks, vs)
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    gen = torch.Generator(device=g.q.device).manual_seed(25)
    cpu_gen = torch.Generator().manual_seed(26)
    full = g.ctx.clone()
    worst = 0.0
    say(f"q8 8-wave stress P={P}")
    for it in range(20):
        g.q = torch.randn(g.q.shape, generator=gen, device=g.q.device).to(torch.float16)
        g.ctx = (torch.randint(0, 1025, (c.B,), generator=cpu_gen, dtype=torch.int32)
                 .to(g.q.device) if it % 2 else full)
        fused = pkv.paged_decode_step_q8(g.q, *gq, g.bt, g.ctx, c.scale, P, workspace=ws)
        again = pkv.paged_decode_step_q8(g.q, *gq, g.bt, g.ctx, c.scale, P, workspace=ws)
        po, pl = pkv.paged_attention_decode_split_q8(g.q, *gq, g.bt, g.ctx, c.scale, P)
        ref3 = pkv.split_reduce(po, pl, g.ctx, P)
        torch.cuda.synchronize()
        assert torch.equal(fused.view(torch.int16), again.view(torch.int16)), f"repeat {it}"
        worst = max(worst, (fused.float() - ref3.float()).abs().max().item())
        _check_workspace_restored(ws)
    assert worst <= 2e-3, worst
