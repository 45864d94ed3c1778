"""kv_cache_append on the GPU against the oracle's scatter: bit-exact over the
whole pool (every byte, NaN sentinels included)."""
import numpy as np
import pytest
import torch

import paged_kv_decode_cache_amd as pkv
from oracle import paged_ref as ref
from gpu_common import DEV, case, needs_gpu, say, to_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]

CONFIGS = ["tiny", "qwen", "sweep:32:4096", "skewed", "long:4:131072"]


def _bytes_equal(got: torch.Tensor, want: np.ndarray) -> bool:
    return np.array_equal(got.cpu().numpy().view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("name", CONFIGS)
def test_append_bit_exact_whole_pool(name):
    c = case(name)
    say(f"append {name}: B={c.B} Hkv={c.Hkv} D={c.D} bs={c.block_size} NB={c.num_blocks}")
    g = to_gpu(c)
    pkv.kv_cache_append(g.k_pool, g.v_pool, g.k_new, g.v_new, g.slots)
    torch.cuda.synchronize()
    kw, vw = ref.kv_cache_append(c.k_pool, c.v_pool, c.k_new, c.v_new, c.slot_mapping)
    assert _bytes_equal(g.k_pool, kw)
    assert _bytes_equal(g.v_pool, vw)


def test_append_skips_negative_and_out_of_range_slots():
    rng = np.random.default_rng(5)
    NB, bs, Hkv, D, N = 7, 16, 2, 128, 12
    kp = rng.standard_normal((NB, bs, Hkv, D)).astype(np.float16)
    vp = rng.standard_normal((NB, bs, Hkv, D)).astype(np.float16)
    kn = rng.standard_normal((N, Hkv, D)).astype(np.float16)
    vn = rng.standard_normal((N, Hkv, D)).astype(np.float16)
    slots = rng.choice(NB * bs, size=N, replace=False).astype(np.int64)
    slots[2] = -1
    slots[5] = -(1 << 40)
    slots[7] = NB * bs            # one past the end: skipped by the kernel
    slots[9] = NB * bs + 1000
    gk = torch.from_numpy(kp).to(DEV)
    gv = torch.from_numpy(vp).to(DEV)
    pkv.kv_cache_append(gk, gv, torch.from_numpy(kn).to(DEV), torch.from_numpy(vn).to(DEV),
                        torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    kw, vw = ref.kv_cache_append(kp, vp, kn, vn, slots)
    assert _bytes_equal(gk, kw) and _bytes_equal(gv, vw)


def test_append_chunked_prefill_fills_whole_blocks():
    """Chunks of 2 blocks' worth of tokens fill 2 more blocks per pass (the
    chunked-prefill block arithmetic, at the library's 16-token blocks)."""
    rng = np.random.default_rng(6)
    NB, bs, Hkv, D = 12, 16, 2, 64
    table = rng.permutation(NB)[:8]
    kp = np.full((NB, bs, Hkv, D), np.nan, dtype=np.float16)
    vp = kp.copy()
    gk = torch.from_numpy(kp).to(DEV)
    gv = torch.from_numpy(vp).to(DEV)
    chunk = 2 * bs
    for i in range(4):
        pos = np.arange(i * chunk, (i + 1) * chunk)
        slots = (table[pos // bs] * bs + pos % bs).astype(np.int64)
        kn = rng.standard_normal((chunk, Hkv, D)).astype(np.float16)
        vn = rng.standard_normal((chunk, Hkv, D)).astype(np.float16)
        pkv.kv_cache_append(gk, gv, torch.from_numpy(kn).to(DEV), torch.from_numpy(vn).to(DEV),
                            torch.from_numpy(slots).to(DEV))
        kp, vp = ref.kv_cache_append(kp, vp, kn, vn, slots)
        torch.cuda.synchronize()
        assert _bytes_equal(gk, kp) and _bytes_equal(gv, vp)
        filled = ~np.isnan(gk.cpu().numpy()).any(axis=(2, 3)).reshape(NB, bs)
        assert int(filled.any(axis=1).sum()) == 2 * (i + 1)


def test_append_zero_tokens_is_noop():
    kp = torch.zeros((2, 16, 1, 64), dtype=torch.float16, device=DEV)
    e = torch.zeros((0, 1, 64), dtype=torch.float16, device=DEV)
    s = torch.zeros((0,), dtype=torch.int64, device=DEV)
    pkv.kv_cache_append(kp, kp.clone(), e, e, s)
    torch.cuda.synchronize()
    assert int(kp.abs().sum()) == 0
