"""A small serving loop driven by the host block allocator: sequences arrive
with a prefill chunk, continue with more chunks or decode steps, and finish;
every step's slots, tables and lengths come from the allocator, the GPU runs
the append + attention calls, and each output is checked against the oracle
on a host mirror of the pools (kept bit-exact with the GPU's)."""
import numpy as np
import pytest
import torch

import paged_kv_decode_cache_amd as pkv
from oracle import paged_ref as ref
from gpu_common import DEV, check_fp16, needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _f16(rng, shape):
    return rng.standard_normal(shape).astype(np.float16)


def test_serving_loop_driven_by_the_allocator():
    rng = np.random.default_rng(530)
    NB, bs, Hq, Hkv, D, S, W, P = 192, 16, 14, 2, 64, 10, 24, 64
    scale = 0.125
    alloc = pkv.BlockAllocator(NB, bs, S, W)
    mk = np.full((NB, bs, Hkv, D), np.nan, dtype=np.float16)
    mv = mk.copy()
    kp, vp = _t(mk), _t(mv)
    live = set()
    workspaces = {}
    steps = {"prefill": 0, "decode": 0, "finished": 0}
    for step in range(40):
        # sequences whose table is full end, and one more now and then
        for s in sorted(live):
            if alloc.context_len(s) >= W * bs:
                alloc.free(s)
                live.discard(s)
                steps["finished"] += 1
        if live and rng.random() < 0.15:
            s = int(rng.choice(sorted(live)))
            alloc.free(s)
            live.discard(s)
            steps["finished"] += 1
        # admissions and continued chunks: one prefill pass
        free_ids = [s for s in range(S) if s not in live]
        new = [int(s) for s in rng.choice(free_ids, size=min(len(free_ids), 2), replace=False)]
        cont = [s for s in sorted(live) if rng.random() < 0.2]
        pre = new + cont
        chunks = [min(int(x), W * bs - alloc.context_len(s))
                  for x, s in zip(rng.integers(1, 120, len(pre)), pre)]
        try:
            qs, slots, tables, lens = alloc.prefill_batch(pre, chunks, W)
        except pkv.NoSpaceError:
            pre = []
        if pre:
            live.update(new)
            T = int(qs[-1])
            q, kn, vn = _f16(rng, (T, Hq, D)), _f16(rng, (T, Hkv, D)), _f16(rng, (T, Hkv, D))
            pkv.kv_cache_append(kp, vp, _t(kn), _t(vn), _t(slots))
            mk, mv = ref.kv_cache_append(mk, mv, kn, vn, slots)
            out = pkv.paged_attention_prefill(_t(q), kp, vp, _t(tables), _t(lens), _t(qs), scale,
                                              max(chunks))
            torch.cuda.synchronize()
            want = ref.paged_attention_prefill(q, mk, mv, tables, lens, qs, scale)
            check_fp16(out, want, f"step {step} prefill {pre}")
            steps["prefill"] += 1
        # one decode step for the other live sequences (fused step)
        dec = [s for s in sorted(live) if s not in pre]
        if not dec:
            continue
        try:
            slots, tables, lens = alloc.decode_batch(dec, W)
        except pkv.NoSpaceError:
            continue
        B = len(dec)
        q, kn, vn = _f16(rng, (B, Hq, D)), _f16(rng, (B, Hkv, D)), _f16(rng, (B, Hkv, D))
        if B not in workspaces:
            workspaces[B] = pkv.StepWorkspace(B, Hq, Hkv, D, pkv.max_partitions_for(W, bs, P),
                                              torch.device(DEV))
        out = pkv.paged_decode_step(_t(q), kp, vp, _t(tables), _t(lens), scale, P,
                                    k_new=_t(kn), v_new=_t(vn), slot_mapping=_t(slots),
                                    workspace=workspaces[B])
        mk, mv = ref.kv_cache_append(mk, mv, kn, vn, slots)
        torch.cuda.synchronize()
        want = ref.paged_attention_decode(q, mk, mv, tables, lens, scale)
        check_fp16(out, want, f"step {step} decode {dec}")
        steps["decode"] += 1
    say(f"serving loop: {steps}, {alloc.num_free} blocks free")
    assert steps["prefill"] >= 10 and steps["decode"] >= 10 and steps["finished"] >= 2
    assert np.array_equal(kp.cpu().numpy().view(np.uint16), mk.view(np.uint16))
    assert np.array_equal(vp.cpu().numpy().view(np.uint16), mv.view(np.uint16))
    for ws in workspaces.values():
        assert int(ws.counters.abs().sum()) == 0
