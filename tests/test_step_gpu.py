"""paged_decode_step (append + split pass + merge in one launch) on the GPU
against the oracle's append followed by its decode."""
import numpy as np
import pytest
import torch

import paged_kv_decode_cache_amd as pkv
import workloads
from oracle import paged_ref as ref
from gpu_common import (PARTIAL_ATOL, case, check_fp16, host64, needs_gpu, oracle_decode,
                        oracle_full, say, to_gpu)

pytestmark = [pytest.mark.gpu, needs_gpu]


def _step(g, c, P, ws=None, append=True, want_lse=True, launch=None):
    kw = dict(k_new=g.k_new, v_new=g.v_new, slot_mapping=g.slots) if append else {}
    return pkv.paged_decode_step(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, c.scale, P, workspace=ws,
                                 want_lse=want_lse, launch=launch, **kw)


def _oracle_step(c, seqs=None):
    kp, vp = ref.kv_cache_append(c.k_pool, c.v_pool, c.k_new, c.v_new, c.slot_mapping)
    out, lse = ref.paged_attention_decode(c.q, kp, vp, c.block_tables, c.context_lens, c.scale,
                                          return_lse=True, seqs=seqs)
    return out, lse, kp, vp


def _check_workspace_restored(ws):
    """Every call leaves the partials and the counters zero ("not
    written"), ready for the next call."""
    assert int(ws.counters.abs().sum()) == 0
    assert bool((ws.partial_out.view(torch.int32) == 0).all())
    assert bool((ws.partial_lse.view(torch.int32) == 0).all())


def _check_lse(got, want, rows=None):
    g = host64(got)
    w = np.asarray(want)
    if rows is not None:
        g, w = g[rows], w[rows]
    assert np.array_equal(np.isneginf(g), np.isneginf(w))
    fin = np.isfinite(w)
    if fin.any():
        assert float(np.abs(g[fin] - w[fin]).max()) <= PARTIAL_ATOL


@pytest.mark.parametrize("name,P", [("tiny", 16), ("tiny", 64), ("qwen", 512), ("qwen", 128),
                                    ("sweep:32:4096", 512), ("sweep:1:128", 512),
                                    ("sweep:8:2048", 256), ("long:1:32768", 512),
                                    ("long:4:32768", 2048), ("long:4:32768", 1024),
                                    ("long:4:32768", 512),
                                    # 8-wave defaults on small grids (8 and 16 partitions)
                                    ("sweep:8:4096", 256), ("sweep:1:4096", 256),
                                    ("sweep:8:4096", 512)])
def test_step_matches_append_then_decode(name, P):
    c = case(name)
    say(f"step {name} P={P}")
    g = to_gpu(c)
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    out, lse = _step(g, c, P, ws)
    torch.cuda.synchronize()
    want, want_lse, kp, vp = _oracle_step(c)
    check_fp16(out, want, f"step {name}")
    _check_lse(lse, want_lse)
    assert np.array_equal(g.k_pool.cpu().numpy().view(np.uint16), kp.view(np.uint16))
    assert np.array_equal(g.v_pool.cpu().numpy().view(np.uint16), vp.view(np.uint16))
    _check_workspace_restored(ws)


@pytest.mark.parametrize("name,grid", [("skewed", "auto"), ("skewed", "compact"),
                                       ("long:4:131072", "auto")])
def test_step_full_size(name, grid):
    """Full-size launches, every sequence against the oracle's append +
    decode."""
    c = case(name)
    P = 512
    say(f"step {name} grid={grid} (all {c.B} sequences)")
    g = to_gpu(c)
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    out, lse = _step(g, c, P, ws, launch=dict(grid=grid))
    torch.cuda.synchronize()
    want, want_lse = oracle_full(name, appended=True)
    check_fp16(out, want, f"step {name} {grid}")
    _check_lse(lse, want_lse)
    _check_workspace_restored(ws)


def test_step_compact_grid_large_ragged_batch():
    """The fused step on the compact grid with 300 ragged sequences (empty
    ones write zeros), every sequence against the oracle's append + decode."""
    rng = np.random.default_rng(134)
    lens = rng.integers(0, 2001, 300).tolist()
    lens[0], lens[1], lens[299] = 0, 2000, 1
    c = workloads.custom_case("step_compact_300", B=300, Hq=14, Hkv=2, D=64, block_size=16,
                              lens=lens, seed=135)
    g = to_gpu(c)
    P = 128
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    out, lse = _step(g, c, P, ws, launch=dict(grid="compact"))
    torch.cuda.synchronize()
    want, want_lse, kp, vp = _oracle_step(c)
    check_fp16(out, want, "step compact B=300")
    _check_lse(lse, want_lse)
    assert np.array_equal(g.k_pool.cpu().numpy().view(np.uint16), kp.view(np.uint16))
    _check_workspace_restored(ws)


def test_step_repeated_calls_reuse_counters():
    """Three steps in a row on one workspace (counters reset each time), the
    second and third with other queries and shorter contexts."""
    c = case("qwen")
    P = 256
    g = to_gpu(c)
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    out1 = _step(g, c, P, ws, want_lse=False).clone()
    torch.cuda.synchronize()
    want, _, _, _ = _oracle_step(c)
    check_fp16(out1, want, "step call 1")
    rng = np.random.default_rng(7)
    for k in (2, 3):
        q2 = (rng.standard_normal(c.q.shape) * 0.5).astype(np.float16)
        ctx2 = np.maximum(c.context_lens - 100 * k, 1).astype(np.int32)
        g.q = torch.from_numpy(q2).to(g.q.device)
        g.ctx = torch.from_numpy(ctx2).to(g.q.device)
        out2 = _step(g, c, P, ws, append=False, want_lse=False)
        torch.cuda.synchronize()
        kp, vp = ref.kv_cache_append(c.k_pool, c.v_pool, c.k_new, c.v_new, c.slot_mapping)
        want2 = ref.paged_attention_decode(q2, kp, vp, c.block_tables, ctx2, c.scale)
        check_fp16(out2, want2, f"step call {k}")
        _check_workspace_restored(ws)


def test_step_without_append_equals_decode():
    c = case("sweep:8:1024")
    g = to_gpu(c)
    out = _step(g, c, 256, append=False, want_lse=False)
    torch.cuda.synchronize()
    want, _ = oracle_decode(c)
    check_fp16(out, want, "step no append")


def test_step_edge_lengths_and_single_partition():
    c = workloads.custom_case("step_edges", B=6, Hq=14, Hkv=2, D=64, block_size=16,
                              lens=[0, 1, 16, 17, 511, 1300], seed=110, q_mult=4.0)
    g = to_gpu(c)
    for P in (16, 512, 2048):
        g2 = to_gpu(c)
        out, lse = _step(g2, c, P)
        torch.cuda.synchronize()
        want, want_lse, kp, _ = _oracle_step(c)
        check_fp16(out, want, f"edges P={P}")
        _check_lse(lse, want_lse)
        assert int((out[0] != 0).sum()) == 0
        assert np.array_equal(g2.k_pool.cpu().numpy().view(np.uint16), kp.view(np.uint16))


def test_step_slot_elsewhere_or_skipped():
    """A new token whose slot is not its position's slot in the table is
    written there, and this step's attention keeps the pool's row at position
    ctx-1 (no substitution); a negative slot writes nothing.  The slots used
    are in blocks no table references, so the expected attention is the plain
    decode over the pool as given."""
    c = workloads.custom_case("step_elsewhere", B=4, Hq=14, Hkv=2, D=64, block_size=16,
                              lens=[5, 300, 1024, 77], seed=112)
    bs = c.block_size
    used = set(c.block_tables[c.block_tables >= 0].tolist())
    spare = [blk for blk in range(c.num_blocks) if blk not in used]
    assert len(spare) >= 2
    slots = np.array([spare[0] * bs + 3, -1, spare[1] * bs + bs - 1, -1], dtype=np.int64)
    for P in (64, 2048):
        g = to_gpu(c)
        g.slots = torch.from_numpy(slots).to(g.q.device)
        out, lse = _step(g, c, P)
        torch.cuda.synchronize()
        want, want_lse = ref.paged_attention_decode(c.q, c.k_pool, c.v_pool, c.block_tables,
                                                    c.context_lens, c.scale, return_lse=True)
        check_fp16(out, want, f"slot elsewhere P={P}")
        _check_lse(lse, want_lse)
        kp, vp = ref.kv_cache_append(c.k_pool, c.v_pool, c.k_new, c.v_new, slots)
        assert np.array_equal(g.k_pool.cpu().numpy().view(np.uint16), kp.view(np.uint16))
        assert np.array_equal(g.v_pool.cpu().numpy().view(np.uint16), vp.view(np.uint16))


@pytest.mark.parametrize("Hq,Hkv,D,bs", [(16, 1, 128, 32), (32, 8, 128, 16), (4, 4, 64, 64),
                                         (12, 1, 64, 16)])
def test_step_other_shapes(Hq, Hkv, D, bs):
    c = workloads.custom_case("step_shapes", B=4, Hq=Hq, Hkv=Hkv, D=D, block_size=bs,
                              lens=[3, 200, 1000, 2500], seed=111)
    g = to_gpu(c)
    out, lse = _step(g, c, 256)
    torch.cuda.synchronize()
    want, want_lse, _, _ = _oracle_step(c)
    check_fp16(out, want, f"step shapes {Hq}/{Hkv}/{D}/{bs}")
    _check_lse(lse, want_lse)


@pytest.mark.parametrize("name,P", [("sweep:32:1024", 256), ("sweep:32:1024", 64),
                                    ("long:1:32768", 512)])
def test_step_in_hip_graph_replays(name, P):
    """The step is capture-safe: replays of a captured step, with eager work
    and synchronisation between them, all equal the eager result (the direct
    merge at 4 partitions per pair, the merge through LDS at 16, and the
    two-level merge at 64)."""
    c = case(name)
    g = to_gpu(c)
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    out = torch.empty((c.B, c.Hq, c.D), dtype=torch.float16, device=g.q.device)
    eager = _step(g, c, P, ws, want_lse=False).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pkv.paged_decode_step(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, c.scale, P, k_new=g.k_new,
                              v_new=g.v_new, slot_mapping=g.slots, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pkv.paged_decode_step(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, c.scale, P, k_new=g.k_new,
                              v_new=g.v_new, slot_mapping=g.slots, workspace=ws, out=out)
    for rep in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        _check_workspace_restored(ws)
        junk = torch.randn(1024, device=g.q.device).sum()  # eager work between replays
        torch.cuda.synchronize()
        del junk


@pytest.mark.parametrize("waves,subtiles,depth", [(1, 1, 2), (2, 2, 4), (4, 2, 2), (8, 4, 2),
                                                  (4, 1, 4)])
def test_step_launch_shapes(waves, subtiles, depth):
    launch = dict(waves=waves, subtiles=subtiles, depth=depth)
    for name in ("qwen", "tiny"):
        c = case(name)
        g = to_gpu(c)
        out = _step(g, c, 64 if name == "tiny" else 256, want_lse=False, launch=launch)
        torch.cuda.synchronize()
        want, _, _, _ = _oracle_step(c)
        check_fp16(out, want, f"step {name} NW={waves} NS={subtiles} DEPTH={depth}")


def test_step_merge_stress_against_three_launch_path():
    """40 fused steps with new queries and new context lengths each time (so
    the number of partitions per sequence changes between calls); each must
    match the append + split pass + split_reduce path (which has no
    cross-workgroup hand-off) within fp16 tolerance.  A merge that read a
    stale or half-written partial would be off by O(1)."""
    c = case("sweep:32:1024")
    P = 128
    g = to_gpu(c)
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    gen = torch.Generator(device=g.q.device).manual_seed(5)
    cpu_gen = torch.Generator().manual_seed(6)
    full = g.ctx.clone()
    worst = 0.0
    for it in range(40):
        g.q = torch.randn(g.q.shape, generator=gen, device=g.q.device).to(torch.float16)
        if it % 2:
            g.ctx = torch.randint(0, 1025, (c.B,), generator=cpu_gen,
                                  dtype=torch.int32).to(g.q.device)
        else:
            g.ctx = full
        fused = _step(g, c, P, ws, append=False, want_lse=False)
        po, pl = pkv.paged_attention_decode_split(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, c.scale,
                                                  P)
        ref3 = pkv.split_reduce(po, pl, g.ctx, P)
        torch.cuda.synchronize()
        worst = max(worst, (fused.float() - ref3.float()).abs().max().item())
        _check_workspace_restored(ws)
    assert worst <= 2e-3, worst


def test_step_compact_grid_edges_and_churn():
    """The fused step on the compact grid: edge lengths (empty sequences write
    zeros), then 20 steps with new queries and random lengths, each against
    the three-launch path, the workspace restored after every call."""
    c = workloads.custom_case("step_compact", B=6, Hq=14, Hkv=2, D=64, block_size=16,
                              lens=[0, 1, 16, 17, 511, 1300], seed=112, q_mult=4.0,
                              max_blocks=96)
    P = 64
    compact = dict(grid="compact")
    if True:
        g = to_gpu(c)
        ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
        out, lse = _step(g, c, P, ws, launch=compact)
        torch.cuda.synchronize()
        want, want_lse, kp, _ = _oracle_step(c)
        check_fp16(out, want, "compact step edges")
        _check_lse(lse, want_lse)
        assert int((out[0] != 0).sum()) == 0
        assert np.array_equal(g.k_pool.cpu().numpy().view(np.uint16), kp.view(np.uint16))
        _check_workspace_restored(ws)
        gen = torch.Generator(device=g.q.device).manual_seed(8)
        cpu_gen = torch.Generator().manual_seed(9)
        worst = 0.0
        for it in range(20):
            g.q = torch.randn(g.q.shape, generator=gen, device=g.q.device).to(torch.float16)
            g.ctx = torch.randint(0, 96 * 16 + 1, (c.B,), generator=cpu_gen,
                                  dtype=torch.int32).to(g.q.device)
            fused = _step(g, c, P, ws, append=False, want_lse=False, launch=compact)
            po, pl = pkv.paged_attention_decode_split(g.q, g.k_pool, g.v_pool, g.bt, g.ctx,
                                                      c.scale, P)
            ref3 = pkv.split_reduce(po, pl, g.ctx, P)
            torch.cuda.synchronize()
            worst = max(worst, (fused.float() - ref3.float()).abs().max().item())
            _check_workspace_restored(ws)
        assert worst <= 2e-3, worst


def test_step_wide_merge_large_group():
    """Groups of 16 query heads (the kernel variant without the dual-half
    columns) at long contexts with few workgroups: the step's default launch
    takes 8 waves for the merge.  Against the oracle's append + decode, and
    against an explicit 4-wave launch."""
    c = workloads.custom_case("step_wide_g16", B=2, Hq=32, Hkv=2, D=64, block_size=16,
                              lens=[16384, 9001], seed=150, q_mult=4.0)
    P = 1024  # 16 partitions, grid 2 x 2 x 16 = 64
    say(f"step wide merge G=16 P={P}")
    g = to_gpu(c)
    out, lse = _step(g, c, P)
    torch.cuda.synchronize()
    want, want_lse, kp, _ = _oracle_step(c)
    check_fp16(out, want, "step wide merge G=16")
    _check_lse(lse, want_lse)
    assert np.array_equal(g.k_pool.cpu().numpy().view(np.uint16), kp.view(np.uint16))
    g4 = to_gpu(c)
    out4, _ = _step(g4, c, P, launch=dict(waves=4, subtiles=1, depth=2))
    torch.cuda.synchronize()
    check_fp16(out4, want, "step G=16 at 4 waves")



# Partition counts around every shape of the two-level merge: one level up
# to 16 partitions, then groups of about 8 (17 -> 3 groups of 6/6/5, 128 ->
# 16 groups of 8, 129 -> 16 groups of 9 with a last group of 4, 256 -> 12
# groups of 22 with a last of 14, 1000 -> 9 groups of 112 with a last of 104).
TWO_LEVEL_NP = [1, 2, 15, 16, 17, 18, 23, 24, 25, 33, 64, 65, 127, 128, 129, 200, 255, 256,
                257, 1000]


@pytest.mark.parametrize("P,launch", [(16, None), (64, None), (16, dict(waves=8)),
                                      (64, dict(grid="compact"))])
def test_step_two_level_merge_group_shapes(P, launch):
    """Sequences whose partition counts cross every group boundary of the
    two-level merge (ragged last partitions), against the oracle's append +
    decode, twice on one workspace (other queries and lengths the second
    time); every call leaves the workspace zero, and a repeated call gives
    bit-identical outputs."""
    rng = np.random.default_rng(160)
    nps = [n for n in TWO_LEVEL_NP if n * P <= 16000 or n == 1000 and P == 16]
    lens = [max(1, n * P - int(rng.integers(0, P))) for n in nps]
    c = workloads.custom_case(f"step_two_level_P{P}", B=len(lens), Hq=14, Hkv=2, D=64,
                              block_size=16, lens=lens, seed=161, q_mult=2.0)
    say(f"step two-level merge P={P} launch={launch} partitions={nps}")
    g = to_gpu(c)
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    out, lse = _step(g, c, P, ws, launch=launch)
    torch.cuda.synchronize()
    want, want_lse, kp, vp = _oracle_step(c)
    check_fp16(out, want, f"two-level P={P}")
    _check_lse(lse, want_lse)
    assert np.array_equal(g.k_pool.cpu().numpy().view(np.uint16), kp.view(np.uint16))
    _check_workspace_restored(ws)
    # shorter contexts and new queries: other group shapes on the same workspace
    q2 = (rng.standard_normal(c.q.shape) * 2.0).astype(np.float16)
    ctx2 = np.maximum(c.context_lens - rng.integers(0, 4 * P, c.B), 0).astype(np.int32)
    g.q = torch.from_numpy(q2).to(g.q.device)
    g.ctx = torch.from_numpy(ctx2).to(g.q.device)
    out2 = _step(g, c, P, ws, append=False, want_lse=False, launch=launch).clone()
    out3 = _step(g, c, P, ws, append=False, want_lse=False, launch=launch)
    torch.cuda.synchronize()
    want2 = ref.paged_attention_decode(q2, kp, vp, c.block_tables, ctx2, c.scale)
    check_fp16(out2, want2, f"two-level P={P} second call")
    assert torch.equal(out2.view(torch.int16), out3.view(torch.int16))
    _check_workspace_restored(ws)


@pytest.mark.parametrize("Hq,Hkv,D,bs", [(32, 2, 64, 16), (32, 2, 128, 16), (16, 4, 128, 32)])
def test_step_two_level_merge_other_shapes(Hq, Hkv, D, bs):
    """The two-level merge with groups of 16 heads (no dual columns; at
    head_dim 128 one merge thread set spans the whole workgroup) and with
    head_dim 128 at block size 32: partition counts on both sides of the
    group boundaries, against the oracle's append + decode, workspace zero
    afterwards."""
    P = 2 * bs
    rng = np.random.default_rng(170 + D + Hq)
    nps = [1, 17, 33, 64, 129, 200]
    lens = [max(1, n * P - int(rng.integers(0, P))) for n in nps]
    c = workloads.custom_case(f"step_two_level_G{Hq // Hkv}_D{D}", B=len(lens), Hq=Hq, Hkv=Hkv,
                              D=D, block_size=bs, lens=lens, seed=171, q_mult=2.0)
    say(f"step two-level Hq={Hq} Hkv={Hkv} D={D} bs={bs} P={P} partitions={nps}")
    g = to_gpu(c)
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    out, lse = _step(g, c, P, ws)
    torch.cuda.synchronize()
    want, want_lse, kp, _ = _oracle_step(c)
    check_fp16(out, want, f"two-level G={Hq // Hkv} D={D}")
    _check_lse(lse, want_lse)
    assert np.array_equal(g.k_pool.cpu().numpy().view(np.uint16), kp.view(np.uint16))
    _check_workspace_restored(ws)


def test_step_two_level_merge_stress_against_three_launch_path():
    """20 fused steps on one workspace with new queries and random context
    lengths at P=64 (1..100 partitions per sequence, so the launches switch
    between the one- and two-level merges and every group shape), each
    against the append-free three-launch path, the workspace zero after each."""
    rng = np.random.default_rng(190)
    lens = rng.integers(1, 6401, 12).tolist()
    c = workloads.custom_case("step_two_level_stress", B=12, Hq=14, Hkv=2, D=64, block_size=16,
                              lens=lens, seed=191, max_blocks=400)
    P = 64
    g = to_gpu(c)
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    gen = torch.Generator(device=g.q.device).manual_seed(192)
    cpu_gen = torch.Generator().manual_seed(193)
    worst = 0.0
    for it in range(20):
        g.q = torch.randn(g.q.shape, generator=gen, device=g.q.device).to(torch.float16)
        g.ctx = torch.randint(0, 400 * 16 + 1, (c.B,), generator=cpu_gen,
                              dtype=torch.int32).to(g.q.device)
        if it % 5 == 0:
            g.ctx[0] = 400 * 16  # a launch with 100 partitions on one pair
        fused = _step(g, c, P, ws, append=False, want_lse=False)
        po, pl = pkv.paged_attention_decode_split(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, c.scale,
                                                  P)
        ref3 = pkv.split_reduce(po, pl, g.ctx, P)
        torch.cuda.synchronize()
        worst = max(worst, (fused.float() - ref3.float()).abs().max().item())
        _check_workspace_restored(ws)
    assert worst <= 2e-3, worst


# Pairs with 0 to 4 partitions of 256 positions (max_blocks 64: at most 4
# partitions per pair, so every launch takes the direct merge).
DIRECT_LENS = [0, 1, 255, 256, 257, 511, 512, 700, 1023, 1024]


@pytest.mark.parametrize("Hq,Hkv,D,grid", [(14, 2, 64, "auto"), (32, 2, 64, "auto"),
                                           (16, 2, 128, "auto"), (32, 2, 128, "auto"),
                                           (14, 2, 64, "compact")])
def test_step_direct_merge(Hq, Hkv, D, grid):
    """Launches with at most 4 partitions per pair, where each merging thread
    takes every partition of its (head, 4 dims) and writes the output itself:
    groups of 7 and 16 heads, head_dim 64 and 128 (at 16 heads of 128 dims a
    thread takes two (head, 4 dims) slots), the direct and compact grids;
    every sequence against the oracle's append + decode, two calls in a row
    on one workspace, the second bit-identical to a repeat of itself."""
    c = workloads.custom_case("step_direct", B=len(DIRECT_LENS), Hq=Hq, Hkv=Hkv, D=D,
                              block_size=16, lens=DIRECT_LENS, seed=140, max_blocks=64)
    P = 256
    assert c.max_partitions(P) == 4
    g = to_gpu(c)
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    out, lse = _step(g, c, P, ws, launch=dict(grid=grid))
    torch.cuda.synchronize()
    want, want_lse, kp, vp = _oracle_step(c)
    check_fp16(out, want, f"direct merge {Hq}/{Hkv}/{D} {grid}")
    _check_lse(lse, want_lse)
    assert int((out[0] != 0).sum()) == 0
    assert np.array_equal(g.k_pool.cpu().numpy().view(np.uint16), kp.view(np.uint16))
    assert np.array_equal(g.v_pool.cpu().numpy().view(np.uint16), vp.view(np.uint16))
    _check_workspace_restored(ws)
    # a second call (no append) with other queries: the decode of the pool
    # as the first call left it, and a repeat gives the same bits
    g.q = torch.randn(g.q.shape, generator=torch.Generator(device=g.q.device).manual_seed(141),
                      device=g.q.device).to(torch.float16)
    again = _step(g, c, P, ws, append=False, want_lse=False, launch=dict(grid=grid)).clone()
    repeat = _step(g, c, P, ws, append=False, want_lse=False, launch=dict(grid=grid))
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), repeat.view(torch.int16))
    want2 = ref.paged_attention_decode(g.q.cpu().numpy(), kp, vp, c.block_tables,
                                       c.context_lens, c.scale)
    check_fp16(again, want2, f"direct merge second call {Hq}/{Hkv}/{D} {grid}")
    _check_workspace_restored(ws)


def test_step_direct_merge_stress_against_three_launch_path():
    """40 fused steps at 4 partitions per pair (the direct merge) with new
    queries and new context lengths, each against append + split pass +
    split_reduce."""
    c = case("sweep:32:1024")
    P = 256
    assert c.max_partitions(P) == 4
    g = to_gpu(c)
    ws = pkv.StepWorkspace(c.B, c.Hq, c.Hkv, c.D, c.max_partitions(P), g.q.device)
    gen = torch.Generator(device=g.q.device).manual_seed(15)
    cpu_gen = torch.Generator().manual_seed(16)
    full = g.ctx.clone()
    worst = 0.0
    for it in range(40):
        g.q = torch.randn(g.q.shape, generator=gen, device=g.q.device).to(torch.float16)
        g.ctx = (torch.randint(0, 1025, (c.B,), generator=cpu_gen, dtype=torch.int32)
                 .to(g.q.device) if it % 2 else full)
        fused = _step(g, c, P, ws, append=False, want_lse=False)
        po, pl = pkv.paged_attention_decode_split(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, c.scale,
                                                  P)
        ref3 = pkv.split_reduce(po, pl, g.ctx, P)
        torch.cuda.synchronize()
        worst = max(worst, (fused.float() - ref3.float()).abs().max().item())
        _check_workspace_restored(ws)
    assert worst <= 2e-3, worst
