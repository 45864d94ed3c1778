"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin from ``test_oracle.py`` fails for every one of them."""
import numpy as np
import pytest

from oracle import paged_ref as ref
import test_oracle as pins


def _attend_factory(kind):
    def attend(q, K, V, scale):
        G, D = q.shape
        n = K.shape[0]
        if n == 0:
            return np.zeros((G, D)), np.full(G, -np.inf)
        s = (q @ K.T) if kind == "no_scale" else scale * (q @ K.T)
        if kind == "keys_as_values":
            V = K
        m = s.max(axis=1, keepdims=True)
        e = np.exp(-(s - m)) if kind == "sign" else np.exp(s - m)
        if kind == "sign":
            e = e / e.max(axis=1, keepdims=True)
        l = e.sum(axis=1, keepdims=True)
        out = (e @ V) if kind == "no_norm" else (e @ V) / l
        lse = (m + (l if kind == "lse_no_log" else np.log(l)))[:, 0]
        if kind == "drop_last":
            o2, _ = ref_attend_orig(q, K[:-1], V[:-1], scale) if n > 1 else (out, None)
            out = o2
        return out, lse
    return attend


ref_attend_orig = ref.attend


def _gather_factory(kind):
    orig = ref.gather_sequence_kv

    def gather(pool, table_row, n, block_size, kvh):
        t = np.arange(n, dtype=np.int64)
        if kind == "offset_shift":
            phys = table_row[t // block_size].astype(np.int64)
            off = (t + 1) % block_size
        elif kind == "swapped_index":
            phys = table_row[(t % block_size) % len(table_row)].astype(np.int64)
            off = (t // block_size) % block_size
        elif kind == "identity_table":
            phys = (t // block_size)
            off = t % block_size
        else:
            return orig(pool, table_row, n, block_size, kvh)
        return pool[phys, off, kvh, :].astype(np.float64)
    return gather


def _merge_factory(kind):
    def merge(outs, lses):
        outs = np.asarray(outs, dtype=np.float64)
        lses = np.asarray(lses, dtype=np.float64)
        if lses.size == 0 or np.all(np.isneginf(lses)):
            return np.zeros(outs.shape[-1]), -np.inf
        mx = lses[np.isfinite(lses)].max()
        if kind == "sign":
            w = np.where(np.isneginf(lses), 0.0, np.exp(mx - lses))
        else:  # unweighted
            w = np.where(np.isneginf(lses), 0.0, 1.0)
        total = w.sum()
        L = mx + np.log(total)
        out = (w[:, None] * np.where(np.isneginf(lses)[:, None], 0.0, outs)).sum(0) / total
        return out, L
    return merge


def _append_transposed(k_pool, v_pool, k_new, v_new, slot_mapping):
    kp, vp = k_pool.copy(), v_pool.copy()
    nb, bs = kp.shape[:2]
    for i, s in enumerate(np.asarray(slot_mapping)):
        if s < 0:
            continue
        blk, off = int(s) % nb, (int(s) // nb) % bs      # wrong decomposition
        kp[blk, off] = k_new[i]
        vp[blk, off] = v_new[i]
    return kp, vp


def _append_no_skip(k_pool, v_pool, k_new, v_new, slot_mapping):
    kp, vp = k_pool.copy(), v_pool.copy()
    fk = kp.reshape(-1, *kp.shape[2:])
    fv = vp.reshape(-1, *vp.shape[2:])
    s = np.asarray(slot_mapping, dtype=np.int64)
    fk[s] = k_new                      # negative slot writes the last row
    fv[s] = v_new
    return kp, vp


def _append_wraps_past_end(k_pool, v_pool, k_new, v_new, slot_mapping):
    kp, vp = k_pool.copy(), v_pool.copy()
    nb, bs = kp.shape[:2]
    for i, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if s < 0:
            continue
        s = int(s) % (nb * bs)         # a slot past the pool wraps instead of being skipped
        kp[s // bs, s % bs] = k_new[i]
        vp[s // bs, s % bs] = v_new[i]
    return kp, vp


def _split_factory(kind):
    orig = ref.paged_attention_decode_split

    def split(q, k_pool, v_pool, block_tables, context_lens, scale, partition_size,
              max_partitions):
        po, pl = orig(q, k_pool, v_pool, block_tables, context_lens, scale,
                      partition_size, max_partitions)
        if kind == "lse_log2":
            pl = pl / np.log(2.0)
        return po, pl
    return split


def _prefill_factory(kind):
    """The prefill oracle with one planted mistake in its causal bookkeeping."""
    def prefill(q, k_pool, v_pool, block_tables, context_lens, query_start, scale,
                return_lse=False, seqs=None):
        T, Hq, D = q.shape
        _, bs, Hkv, _ = k_pool.shape
        sc = ref.fp32_scale(scale)
        out = np.zeros((T, Hq, D))
        lse = np.full((T, Hq), -np.inf)
        B = len(context_lens)
        n_first = int(query_start[1] - query_start[0]) if B else 0
        for b in (range(B) if seqs is None else seqs):
            r0, r1 = int(query_start[b]), int(query_start[b + 1])
            if kind == "rows_by_equal_chunks":
                r0, r1 = b * n_first, (b + 1) * n_first
            n, ctx = r1 - r0, int(context_lens[b])
            for kvh in range(Hkv):
                heads = ref.heads_of_kv_head(kvh, Hq, Hkv)
                K = ref.gather_sequence_kv(k_pool, block_tables[b], ctx, bs, kvh)
                V = ref.gather_sequence_kv(v_pool, block_tables[b], ctx, bs, kvh)
                for i in range(n):
                    pos = i if kind == "top_left_causal" else ctx - n + i
                    if pos < 0 or r0 + i >= T:
                        continue
                    end = {"excludes_itself": pos, "sees_next_token": pos + 2,
                           "not_causal": ctx}.get(kind, pos + 1)
                    o, ls = ref.attend(q[r0 + i, heads].astype(np.float64), K[:end], V[:end], sc)
                    out[r0 + i, heads] = o
                    lse[r0 + i, heads] = ls
        return (out, lse) if return_lse else out
    return prefill


def _q8_factory(kind):
    """The 8-bit quantiser with one planted mistake."""
    def quantize(x16):
        x = np.asarray(x16).astype(np.float32)
        amax = np.max(np.abs(x), axis=-1)
        if kind == "per_tensor_amax":
            amax = np.full_like(amax, np.max(np.abs(x)))
        nz = amax > 0
        inv = np.zeros_like(amax)
        inv[nz] = (np.float32(1.0) if kind == "no_127" else np.float32(127.0)) / amax[nz]
        y = x * inv[..., None]
        codes = np.trunc(y) if kind == "truncates" else np.rint(y)
        codes = np.clip(codes, -128 if kind == "clip_128" else -127, 127).astype(np.int8)
        scales = (amax / np.float32(127.0)).astype(np.float32)
        return codes, scales
    return quantize


MUTANTS = {
    "gqa_modulo": ("kv_head_of", lambda h, Hq, Hkv: h % Hkv),
    "no_scale": ("attend", _attend_factory("no_scale")),
    "softmax_sign": ("attend", _attend_factory("sign")),
    "no_normalise": ("attend", _attend_factory("no_norm")),
    "keys_as_values": ("attend", _attend_factory("keys_as_values")),
    "lse_without_log": ("attend", _attend_factory("lse_no_log")),
    "drops_last_token": ("attend", _attend_factory("drop_last")),
    "offset_shift": ("gather_sequence_kv", _gather_factory("offset_shift")),
    "swapped_block_offset": ("gather_sequence_kv", _gather_factory("swapped_index")),
    "ignores_block_table": ("gather_sequence_kv", _gather_factory("identity_table")),
    "merge_sign": ("merge_partitions", _merge_factory("sign")),
    "merge_unweighted": ("merge_partitions", _merge_factory("unweighted")),
    "append_transposed_slot": ("kv_cache_append", _append_transposed),
    "append_no_skip": ("kv_cache_append", _append_no_skip),
    "append_wraps_past_end": ("kv_cache_append", _append_wraps_past_end),
    "split_lse_base2": ("paged_attention_decode_split", _split_factory("lse_log2")),
    "scale_not_fp32": ("fp32_scale", lambda s: float(s) * (1 + 1e-7)),
    "q8_per_tensor_amax": ("quantize_rows_q8", _q8_factory("per_tensor_amax")),
    "q8_missing_127": ("quantize_rows_q8", _q8_factory("no_127")),
    "q8_truncates": ("quantize_rows_q8", _q8_factory("truncates")),
    "prefill_excludes_itself": ("paged_attention_prefill", _prefill_factory("excludes_itself")),
    "prefill_sees_next_token": ("paged_attention_prefill", _prefill_factory("sees_next_token")),
    "prefill_not_causal": ("paged_attention_prefill", _prefill_factory("not_causal")),
    "prefill_top_left_causal": ("paged_attention_prefill", _prefill_factory("top_left_causal")),
    "prefill_rows_by_equal_chunks": ("paged_attention_prefill",
                                     _prefill_factory("rows_by_equal_chunks")),
}


def _fails(fn):
    try:
        fn()
    except (AssertionError, IndexError, ValueError, FloatingPointError):
        return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_a_pin_catches_mutant(name, monkeypatch):
    attr, repl = MUTANTS[name]
    monkeypatch.setattr(ref, attr, repl)
    caught = [i for i, p in enumerate(pins.ALL_PINS) if _fails(p)]
    assert caught, f"no pin catches the planted mistake {name!r}"


def test_unmutated_oracle_passes_every_pin():
    assert not [i for i, p in enumerate(pins.ALL_PINS) if _fails(p)]
