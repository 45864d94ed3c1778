"""Parity of every workload configuration, every decode path, against the
fp64 oracle, with the measured errors printed (one line per config and path,
on stderr): unsplit decode, split pass + merge (P=512), and the fused step
with its append.  Full-size launches, every sequence compared."""
import numpy as np
import pytest
import torch

import paged_kv_decode_cache_amd as pkv
import workloads
from oracle import paged_ref as ref
from gpu_common import case, check_fp16, needs_gpu, oracle_full, say, to_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]

CONFIGS = (["tiny", "qwen"]
           + [f"sweep:{B}:{c}" for B in workloads.SWEEP_B for c in workloads.SWEEP_CTX]
           + ["skewed"] + [f"long:{B}:{c}" for B, c in workloads.LONG_POINTS]
           # values drawn as fp32 normals rounded to fp16, tails uncut
           + ["qwen+fp32", "sweep:32:4096+fp32", "long:1:32768+fp32"])


@pytest.mark.parametrize("name", CONFIGS)
def test_config_parity_all_paths(name):
    c = case(name)
    P = 16 if name == "tiny" else 512
    g = to_gpu(c)
    dec = pkv.paged_attention_decode(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, c.scale)
    po, pl = pkv.paged_attention_decode_split(g.q, g.k_pool, g.v_pool, g.bt, g.ctx, c.scale, P)
    spl = pkv.split_reduce(po, pl, g.ctx, P)
    torch.cuda.synchronize()
    want, _ = oracle_full(name)
    errs = {"decode": check_fp16(dec, want, f"{name} decode"),
            "split": check_fp16(spl, want, f"{name} split")}
    # fused step: the append of each sequence's new token at ctx-1, then decode
    g2 = to_gpu(c)
    step = pkv.paged_decode_step(g2.q, g2.k_pool, g2.v_pool, g2.bt, g2.ctx, c.scale, P,
                                 k_new=g2.k_new, v_new=g2.v_new, slot_mapping=g2.slots)
    torch.cuda.synchronize()
    want_step, _ = oracle_full(name, appended=True)
    errs["step"] = check_fp16(step, want_step, f"{name} step")
    kp, vp = ref.kv_cache_append(c.k_pool, c.v_pool, c.k_new, c.v_new, c.slot_mapping)
    assert np.array_equal(g2.k_pool.cpu().numpy().view(np.uint16), kp.view(np.uint16))
    assert np.array_equal(g2.v_pool.cpu().numpy().view(np.uint16), vp.view(np.uint16))
    for path, (ma, mr) in errs.items():
        say(f"PARITY {name} {path}: max_abs {ma:.3e} max_rel(|ref|>=0.2) {mr:.3e} "
            f"over all {c.B} sequences")
