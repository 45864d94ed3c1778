"""paged_decode_step_noalloc, the fused decode step on the library's static
scratch, called through the C ABI: on two calls in a row (the second on a
smaller batch) its output and cache write equal those of paged_decode_step
with a caller workspace, bit for bit (same kernels, same summation order),
and both are within the fp16 tolerance of the fp64 oracle's append + decode."""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_decode_cache_amd as pkv
from gpu_common import case, check_fp16, host64, needs_gpu, say, to_gpu
from oracle import paged_ref as ref

pytestmark = [pytest.mark.gpu, needs_gpu]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(g, c, P, out, lse):
    lib = pkv.load_library()
    B, Hq, D = c.q.shape
    NB, bs, Hkv, _ = c.k_pool.shape
    maxb = c.block_tables.shape[1]
    Pm = pkv.max_partitions_for(maxb, bs, P)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.paged_decode_step_noalloc(
        _ptr(out), _ptr(lse), _ptr(g.k_pool), _ptr(g.v_pool), _ptr(g.q), _ptr(g.k_new),
        _ptr(g.v_new), _ptr(g.slots), _ptr(g.bt), _ptr(g.ctx), B, Hq, Hkv, D, bs, NB, maxb, P,
        Pm, float(c.scale), stream)


@pytest.mark.parametrize("calls", [(("qwen", 256), ("tiny", 16)),
                                   (("sweep:32:4096", 1024), ("sweep:8:512", 128)),
                                   # the two-level merge (64 partitions per pair), then a
                                   # smaller one-level call on the same scratch
                                   (("long:1:32768", 512), ("qwen", 256))])
def test_noalloc_step_equals_workspace_step(calls):
    for name, P in calls:
        c = case(name)
        say(f"noalloc step {name} P={P}")
        g_ref, g_na = to_gpu(c), to_gpu(c)
        want_out, want_lse = pkv.paged_decode_step(
            g_ref.q, g_ref.k_pool, g_ref.v_pool, g_ref.bt, g_ref.ctx, c.scale, P,
            k_new=g_ref.k_new, v_new=g_ref.v_new, slot_mapping=g_ref.slots, want_lse=True)
        out = torch.empty_like(want_out)
        lse = torch.empty_like(want_lse)
        assert _noalloc(g_na, c, P, out, lse) == pkv.PKV_OK
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want_out.view(torch.int16)), name
        assert torch.equal(lse.view(torch.int32), want_lse.view(torch.int32)), name
        assert torch.equal(g_na.k_pool.view(torch.int16), g_ref.k_pool.view(torch.int16))
        assert torch.equal(g_na.v_pool.view(torch.int16), g_ref.v_pool.view(torch.int16))
        kp, vp = ref.kv_cache_append(c.k_pool, c.v_pool, c.k_new, c.v_new, c.slot_mapping)
        want, want_l = ref.paged_attention_decode(c.q, kp, vp, c.block_tables, c.context_lens,
                                                  c.scale, return_lse=True)
        check_fp16(out, want, f"noalloc {name}")
        fin = np.isfinite(want_l)
        assert float(np.abs(host64(lse)[fin] - want_l[fin]).max()) <= 2e-4


def test_noalloc_rejects_what_the_scratch_cannot_hold():
    """A call whose workspace exceeds the 16 MiB scratch is refused with
    PKV_ERR_SCRATCH before anything is launched; a fitting call still works."""
    c = case("tiny")
    g = to_gpu(c)
    B, Hq, D = c.q.shape
    NB, bs, Hkv, _ = c.k_pool.shape
    lib = pkv.load_library()
    out = torch.empty((B, Hq, D), dtype=torch.float16, device=g.q.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # 2 x 2 x 70000 partitions x 64 dims x 4 bytes = 71.7 MB of partials
    rc = lib.paged_decode_step_noalloc(
        _ptr(out), None, _ptr(g.k_pool), _ptr(g.v_pool), _ptr(g.q), None, None, None,
        _ptr(g.bt), _ptr(g.ctx), B, Hq, Hkv, D, bs, NB, c.block_tables.shape[1], 16, 70000,
        float(c.scale), stream)
    assert rc == pkv.PKV_ERR_SCRATCH
    assert _noalloc(g, c, 16, out, None) == pkv.PKV_OK
    torch.cuda.synchronize()
