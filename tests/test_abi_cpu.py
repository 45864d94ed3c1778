"""C-ABI checks that need no GPU: the library loads, exports every function
include/pkv.h declares, and rejects invalid arguments with the documented
status before any HIP call (so nothing is launched)."""
import ctypes
import math

import pytest
import torch

import paged_kv_decode_cache_amd as pkv

# Raw-pointer validation calls must never reach a launch on a real device; they
# are host-only checks, so they run only where no GPU is visible.
host_only = pytest.mark.skipif(torch.cuda.is_available(),
                               reason="raw-pointer validation checks run without a GPU")

A16 = 0x10000          # fake, 16-byte aligned "device" addresses (never dereferenced)
B16 = 0x20000
C16 = 0x30000
D16 = 0x40000
E16 = 0x50000
F16 = 0x60000
G16 = 0x70000
H16 = 0x80000
I16 = 0x90000
J16 = 0xA0000
K16 = 0xB0000
L16 = 0xC0000
M16 = 0xD0000


def test_library_exports_every_declared_symbol():
    lib = pkv.load_library()
    names = pkv.declared_functions()
    for expected in ("kv_cache_append", "paged_attention_decode",
                     "paged_attention_decode_split", "split_reduce", "paged_decode_step",
                     "paged_attention_prefill", "pkv_status_string"):
        assert expected in names
    for name in names:
        assert hasattr(lib, name), f"libpkv.so does not export {name}"


def test_status_strings_and_version():
    lib = pkv.load_library()
    assert pkv.status_string(0) == "ok"
    assert "invalid" in pkv.status_string(-1)
    assert "unsupported" in pkv.status_string(-2)
    assert "launch" in pkv.status_string(-3)
    assert pkv.status_string(7) == "unknown status"
    assert lib.pkv_version() >= 100


@host_only
def test_launch_config_validation():
    """A launch shape outside its set is an argument error, decided before
    any HIP call (so it is checkable here); NULL and in-set shapes pass."""
    lib = pkv.load_library()
    args = (A16, B16, C16, D16, E16, F16, 2, 14, 2, 64, 16, 10, 4, 0.125)
    for bad in ((3, 0, 0, 0), (16, 0, 0, 0), (0, 3, 0, 0), (0, 0, 3, 0), (0, 0, 1, 0),
                (0, 0, 0, 3), (0, 0, 0, -1)):
        cfg = pkv.LaunchConfig(*bad)
        assert lib.paged_attention_decode_ex(*args, ctypes.byref(cfg), None) == -1, bad
        assert lib.paged_attention_decode_split_ex(
            A16, B16, C16, D16, E16, F16, G16, 2, 14, 2, 64, 16, 10, 4, 64, 1, 0.125,
            ctypes.byref(cfg), None) == -1, bad
        assert lib.paged_decode_step_ex(
            A16, B16, C16, D16, E16, F16, G16, H16, I16, J16, K16, L16, M16, 2, 14, 2, 64, 16,
            10, 4, 64, 1, 0.125, ctypes.byref(cfg), None) == -1, bad
    empty = (A16, B16, C16, D16, E16, F16, 0, 14, 2, 64, 16, 10, 4, 0.125)
    for good in ((0, 0, 0, 0), (1, 1, 2, 1), (8, 4, 4, 2), (2, 2, 0, 0)):
        cfg = pkv.LaunchConfig(*good)
        assert lib.paged_attention_decode_ex(*empty, ctypes.byref(cfg), None) == 0, good
    assert lib.paged_attention_decode_ex(*empty, None, None) == 0


def _decode(lib, **kw):
    a = dict(out=A16, q=B16, k=C16, v=D16, bt=E16, ctx=F16, B=2, Hq=14, Hkv=2, D=64, bs=16,
             NB=10, maxb=4, scale=0.125)
    a.update(kw)
    return lib.paged_attention_decode(a["out"], a["q"], a["k"], a["v"], a["bt"], a["ctx"], a["B"],
                                      a["Hq"], a["Hkv"], a["D"], a["bs"], a["NB"], a["maxb"],
                                      a["scale"], None)


DECODE_BAD = [
    ("null out", dict(out=None), -1),
    ("null q", dict(q=None), -1),
    ("null pool", dict(k=None), -1),
    ("null table", dict(bt=None), -1),
    ("misaligned q", dict(q=B16 + 2), -1),
    ("misaligned out", dict(out=A16 + 8), -1),
    ("misaligned table", dict(bt=E16 + 2), -1),
    ("negative batch", dict(B=-1), -1),
    ("zero heads", dict(Hq=0), -1),
    ("group not integral", dict(Hq=15), -1),
    ("zero blocks", dict(NB=0), -1),
    ("zero table width", dict(maxb=0), -1),
    ("nan scale", dict(scale=math.nan), -1),
    ("inf scale", dict(scale=math.inf), -1),
    ("head dim 96", dict(D=96), -2),
    ("head dim 256", dict(D=256), -2),
    ("block size 8", dict(bs=8), -2),
    ("block size 24", dict(bs=24), -2),
    ("block size 512", dict(bs=512), -2),
    ("group of 32", dict(Hq=64, Hkv=2), -2),
]


@host_only
@pytest.mark.parametrize("name,kw,code", DECODE_BAD, ids=[d[0] for d in DECODE_BAD])
def test_decode_rejects(name, kw, code):
    assert _decode(pkv.load_library(), **kw) == code


@host_only
def test_decode_batch0_is_noop():
    assert _decode(pkv.load_library(), B=0) == 0


def _split(lib, **kw):
    a = dict(po=A16, pl=B16, q=C16, k=D16, v=E16, bt=F16, ctx=F16 + 0x1000, B=2, Hq=14, Hkv=2,
             D=64, bs=16, NB=10, maxb=4, P=32, Pm=2, scale=0.125)
    a.update(kw)
    return lib.paged_attention_decode_split(a["po"], a["pl"], a["q"], a["k"], a["v"], a["bt"],
                                            a["ctx"], a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"],
                                            a["NB"], a["maxb"], a["P"], a["Pm"], a["scale"], None)


SPLIT_BAD = [
    ("null partial_out", dict(po=None), -1),
    ("null partial_lse", dict(pl=None), -1),
    ("misaligned partial_out", dict(po=A16 + 4), -1),
    ("partition not multiple of block", dict(P=24), -1),
    ("zero partition", dict(P=0), -1),
    ("too few partitions", dict(Pm=1), -1),
    ("zero partitions", dict(Pm=0), -1),
    ("head dim 80", dict(D=80), -2),
]


@host_only
@pytest.mark.parametrize("name,kw,code", SPLIT_BAD, ids=[d[0] for d in SPLIT_BAD])
def test_split_rejects(name, kw, code):
    assert _split(pkv.load_library(), **kw) == code


@host_only
def test_split_batch0_is_noop():
    assert _split(pkv.load_library(), B=0) == 0


def _reduce(lib, **kw):
    a = dict(out=A16, lse=B16, po=C16, pl=D16, ctx=E16, B=2, Hq=14, D=64, P=32, Pm=2)
    a.update(kw)
    return lib.split_reduce(a["out"], a["lse"], a["po"], a["pl"], a["ctx"], a["B"], a["Hq"],
                            a["D"], a["P"], a["Pm"], None)


REDUCE_BAD = [
    ("null out", dict(out=None), -1),
    ("null partials", dict(po=None), -1),
    ("null ctx", dict(ctx=None), -1),
    ("misaligned lse_out", dict(lse=B16 + 2), -1),
    ("zero partition", dict(P=0), -1),
    ("negative batch", dict(B=-3), -1),
    ("head dim 32", dict(D=32), -2),
]


@host_only
@pytest.mark.parametrize("name,kw,code", REDUCE_BAD, ids=[d[0] for d in REDUCE_BAD])
def test_reduce_rejects(name, kw, code):
    assert _reduce(pkv.load_library(), **kw) == code


def _append(lib, **kw):
    a = dict(k=A16, v=B16, kn=C16, vn=D16, slots=E16, N=3, NB=10, bs=16, Hkv=2, D=64)
    a.update(kw)
    return lib.kv_cache_append(a["k"], a["v"], a["kn"], a["vn"], a["slots"], a["N"], a["NB"],
                               a["bs"], a["Hkv"], a["D"], None)


APPEND_BAD = [
    ("null pool", dict(k=None), -1),
    ("null slots", dict(slots=None), -1),
    ("misaligned k_new", dict(kn=C16 + 2), -1),
    ("misaligned slots", dict(slots=E16 + 4), -1),
    ("negative tokens", dict(N=-1), -1),
    ("zero heads", dict(Hkv=0), -1),
    ("head dim 48", dict(D=48), -2),
    ("block size 20", dict(bs=20), -2),
]


@host_only
@pytest.mark.parametrize("name,kw,code", APPEND_BAD, ids=[d[0] for d in APPEND_BAD])
def test_append_rejects(name, kw, code):
    assert _append(pkv.load_library(), **kw) == code


@host_only
def test_append_zero_tokens_is_noop():
    assert _append(pkv.load_library(), N=0) == 0


def _prefill(lib, **kw):
    a = dict(out=A16, q=B16, k=C16, v=D16, bt=E16, ctx=F16, qs=F16 + 0x1000, B=2, maxq=8, Hq=14,
             Hkv=2, D=64, bs=16, NB=10, maxb=4, scale=0.125)
    a.update(kw)
    return lib.paged_attention_prefill(a["out"], a["q"], a["k"], a["v"], a["bt"], a["ctx"],
                                       a["qs"], a["B"], a["maxq"], a["Hq"], a["Hkv"], a["D"],
                                       a["bs"], a["NB"], a["maxb"], a["scale"], None)


PREFILL_BAD = [
    ("null out", dict(out=None), -1),
    ("null query_start", dict(qs=None), -1),
    ("misaligned query_start", dict(qs=F16 + 0x1002), -1),
    ("misaligned out", dict(out=A16 + 4), -1),
    ("negative max_query_len", dict(maxq=-1), -1),
    ("nan scale", dict(scale=math.nan), -1),
    ("head dim 96", dict(D=96), -2),
    ("group of 32", dict(Hq=64, Hkv=2), -2),
]


@host_only
@pytest.mark.parametrize("name,kw,code", PREFILL_BAD, ids=[d[0] for d in PREFILL_BAD])
def test_prefill_rejects(name, kw, code):
    assert _prefill(pkv.load_library(), **kw) == code


@host_only
def test_prefill_empty_is_noop():
    lib = pkv.load_library()
    assert _prefill(lib, B=0) == 0
    assert _prefill(lib, maxq=0) == 0


def _prefill_split(lib, **kw):
    a = dict(po=0xA0000, pl=0xB0000, rl=0xC0000, q=B16, k=C16, v=D16, bt=E16, ctx=F16,
             qs=F16 + 0x1000, B=2, maxq=8, Hq=14, Hkv=2, D=64, bs=16, NB=10, maxb=4, P=32,
             Pm=2, scale=0.125)
    a.update(kw)
    return lib.paged_attention_prefill_split(a["po"], a["pl"], a["rl"], a["q"], a["k"], a["v"],
                                             a["bt"], a["ctx"], a["qs"], a["B"], a["maxq"],
                                             a["Hq"], a["Hkv"], a["D"], a["bs"], a["NB"],
                                             a["maxb"], a["P"], a["Pm"], a["scale"], None)


PREFILL_SPLIT_BAD = [
    ("null partials", dict(po=None), -1),
    ("null row lengths", dict(rl=None), -1),
    ("misaligned partials", dict(po=0xA0000 + 4), -1),
    ("misaligned row lengths", dict(rl=0xC0000 + 2), -1),
    ("null query_start", dict(qs=None), -1),
    ("partition not a block multiple", dict(P=24), -1),
    ("partitions do not cover the table", dict(Pm=1), -1),
    ("negative max_query_len", dict(maxq=-1), -1),
    ("head dim 96", dict(D=96), -2),
]


@host_only
@pytest.mark.parametrize("name,kw,code", PREFILL_SPLIT_BAD, ids=[d[0] for d in PREFILL_SPLIT_BAD])
def test_prefill_split_rejects(name, kw, code):
    assert _prefill_split(pkv.load_library(), **kw) == code


@host_only
def test_prefill_split_empty_is_noop():
    lib = pkv.load_library()
    assert _prefill_split(lib, B=0) == 0
    assert _prefill_split(lib, maxq=0) == 0


def _step(lib, **kw):
    a = dict(out=A16, lse=None, k=C16, v=D16, q=B16, kn=0x70000, vn=0x80000, slots=0x90000,
             bt=E16, ctx=F16, po=0xA0000, pl=0xB0000, cnt=0xC0000, B=2, Hq=14, Hkv=2, D=64,
             bs=16, NB=10, maxb=4, P=32, Pm=2, scale=0.125)
    a.update(kw)
    return lib.paged_decode_step(a["out"], a["lse"], a["k"], a["v"], a["q"], a["kn"], a["vn"],
                                 a["slots"], a["bt"], a["ctx"], a["po"], a["pl"], a["cnt"],
                                 a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["NB"], a["maxb"],
                                 a["P"], a["Pm"], a["scale"], None)


STEP_BAD = [
    ("null out", dict(out=None), -1),
    ("null partials", dict(po=None), -1),
    ("null counters", dict(cnt=None), -1),
    ("misaligned partials", dict(po=0xA0000 + 4), -1),
    ("misaligned new key", dict(kn=0x70000 + 2), -1),
    ("partition not a block multiple", dict(P=24), -1),
    ("partitions do not cover the table", dict(Pm=1), -1),
    # one resource spans a (sequence, KV head)'s partials: G * Pm * D * 4 < 2^30
    ("partials of a pair past 2^30 bytes", dict(Hq=16, Hkv=1, D=128, maxb=131072, P=16,
                                                Pm=131072), -2),
]


@host_only
@pytest.mark.parametrize("name,kw,code", STEP_BAD, ids=[c[0] for c in STEP_BAD])
def test_step_rejects(name, kw, code):
    assert _step(pkv.load_library(), **kw) == code


@host_only
def test_step_batch0_is_noop():
    assert _step(pkv.load_library(), B=0) == 0


def _step_q8(lib, **kw):
    a = dict(out=A16, lse=None, kc=C16, vc=D16, ks=0x50000, vs=0x60000, q=B16, kn=0x70000,
             vn=0x80000, slots=0x90000, bt=E16, ctx=F16, po=0xA0000, pl=0xB0000, cnt=0xC0000,
             B=2, Hq=14, Hkv=2, D=64, bs=16, NB=10, maxb=4, P=32, Pm=2, scale=0.125)
    a.update(kw)
    return lib.paged_decode_step_q8(a["out"], a["lse"], a["kc"], a["vc"], a["ks"], a["vs"],
                                    a["q"], a["kn"], a["vn"], a["slots"], a["bt"], a["ctx"],
                                    a["po"], a["pl"], a["cnt"], a["B"], a["Hq"], a["Hkv"],
                                    a["D"], a["bs"], a["NB"], a["maxb"], a["P"], a["Pm"],
                                    a["scale"], None)


STEP_Q8_BAD = STEP_BAD + [
    ("null scales", dict(ks=None), -1),
    ("misaligned scales", dict(vs=0x60000 + 4), -1),
    ("head_dim 96", dict(D=96), -2),
]


@host_only
@pytest.mark.parametrize("name,kw,code", STEP_Q8_BAD, ids=[c[0] for c in STEP_Q8_BAD])
def test_step_q8_rejects(name, kw, code):
    assert _step_q8(pkv.load_library(), **kw) == code


@host_only
def test_step_q8_batch0_is_noop():
    assert _step_q8(pkv.load_library(), B=0) == 0


def test_binding_rejects_cpu_tensors():
    q = torch.zeros((1, 2, 64), dtype=torch.float16)
    kp = torch.zeros((2, 16, 1, 64), dtype=torch.float16)
    bt = torch.zeros((1, 1), dtype=torch.int32)
    ctx = torch.ones(1, dtype=torch.int32)
    with pytest.raises(ValueError):
        pkv.paged_attention_decode(q, kp, kp, bt, ctx, 0.125)


def test_binding_rejects_wrong_dtype():
    q = torch.zeros((1, 2, 64), dtype=torch.float32)
    kp = torch.zeros((2, 16, 1, 64), dtype=torch.float16)
    bt = torch.zeros((1, 1), dtype=torch.int32)
    ctx = torch.ones(1, dtype=torch.int32)
    with pytest.raises(TypeError):
        pkv.paged_attention_decode(q, kp, kp, bt, ctx, 0.125)


@host_only
def test_step_noalloc_rejects_oversize_and_bad_args():
    """paged_decode_step_noalloc: argument errors as paged_decode_step, and a
    workspace larger than its static scratch gives PKV_ERR_SCRATCH, all
    decided before any HIP call."""
    lib = pkv.load_library()
    base = dict(out=A16, lse=None, k=B16, v=C16, q=D16, kn=None, vn=None, slots=None, bt=E16,
                ctx=F16, B=2, Hq=14, Hkv=2, D=64, bs=16, NB=10, maxb=4, P=64, Pm=1, scale=0.125)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return lib.paged_decode_step_noalloc(
            a["out"], a["lse"], a["k"], a["v"], a["q"], a["kn"], a["vn"], a["slots"], a["bt"],
            a["ctx"], a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["NB"], a["maxb"], a["P"],
            a["Pm"], a["scale"], None)
    assert call(B=0) == 0
    assert call(out=None) == -1
    assert call(P=24) == -1                      # not a multiple of block_size
    assert call(Pm=0) == -1
    assert call(D=96) == -2
    # 4096 x 32 x 256 partitions x 128 dims x 4 bytes = 17 GB of partials
    assert call(B=4096, Hq=32, Hkv=8, D=128, maxb=2048, P=256, Pm=128) == pkv.PKV_ERR_SCRATCH
    assert "scratch" in pkv.status_string(pkv.PKV_ERR_SCRATCH)
