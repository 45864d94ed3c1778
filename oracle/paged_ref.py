"""fp64 CPU oracle for paged KV-cache decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only the test suite, the smoke check and the benchmark's CPU
baseline leg may use it.  It shares no code with the HIP kernels (no common
headers, helpers, tables or pre/post-processing); the only thing both sides
consume is the seeded input generator in ``workloads/``.

What it computes, and where that comes from
-------------------------------------------
* Paged cache layout: fixed-size blocks plus one block table per sequence
  (nanoserve write-up, section "What I built", paged KV cache item).  The pool
  layout is ``[num_blocks, block_size, num_kv_heads, head_dim]``, one pool for
  K and one for V.
* Decode attention: one new query token per sequence attends over all of its
  cached positions, reached through the block table (same section, fused
  paged-attention decode item).  The write-up compares that kernel against a
  "gather the K/V, then run dense scaled-dot-product attention" path (section
  "Results"); the plain definition of what both compute is

      K_b[t] = K_pool[table[b, t // bs], t % bs, kvh(h)]      t < ctx_b
      out[b, h] = softmax(scale * K_b q[b, h]) @ V_b

  and that definition is what this module writes out, in fp64, from the fp16
  inputs (fp16 -> fp64 is exact).  Online softmax and the split-context merge
  reach the same value up to rounding order, so there is nothing else to model.
* Split-context decode ("flash-decoding style" arm, author's post thread, the
  Day 74 post): each sequence's positions are cut into partitions of
  ``partition_size`` tokens; each partition yields its normalised output and
  the natural-log log-sum-exp of its logits; the merge weights partition p by
  exp(lse_p - LSE).  The pages name the arm but not the merge; the LSE-weighted
  merge is the plainest exact reading.
* Chunked prefill (Inference Engineering, Day 12 post on chunked prefill in
  vLLM): a long prompt is split into chunks that are processed and written to
  the cache one pass at a time, as a runtime optimisation only.  So a chunk's
  token at position p attends to positions 0..p of its sequence (the cached
  prefix and the chunk's earlier tokens), exactly as unchunked causal
  attention over the whole prompt would.  A call carries, per sequence, the
  chunk's n query rows; the chunk holds the last n of the sequence's
  context_lens positions (its K/V already written), so row i sits at position
  ctx - n + i.
* Cache write: each step writes the new token's K and V into its slot of the
  pool (Inference Engineering, Day 11 post on how vLLM works: the executor
  updates the cache with the new key and value vectors).  Slots are addressed
  by ``slot = physical_block * block_size + offset``; a negative slot is
  skipped.

* 8-bit cache (the pages mention only another system's q8 KV cache: Gemma
  on llama.cpp with 8-bit K/V, in the post on an RTX 4090, and give no
  format).  This library's format: every (token, KV head) row of D values is
  stored as int8 codes with one fp32 scale, quantised when written:
  amax = max |x| (the fp16 values widened to fp32), inv = 127 / amax and
  code = rint(x * inv) (fp32 division and multiply, nearest-even), clipped
  to [-127, 127]; scale = amax / 127; a row of zeros has codes 0 and scale 0.
  Its value is code * scale.  Attention over an 8-bit cache is the plain
  definition above applied to those values.

Readings where the pages are silent:
* GQA: query head h uses KV head ``h // (Hq // Hkv)`` (contiguous groups).
* ``context_lens`` counts the attended positions, including the token the
  same step appended.
* ctx == 0 gives a zero output and lse = -inf.
* The scale the kernel receives is an fp32 value; the oracle uses that fp32
  value widened to fp64 and applies it to the fp64 dot product.

Every function here is pinned by ``tests/test_oracle.py`` against things other
than itself (torch's fp64 SDPA on contiguous K/V, closed forms, block-id
permutation invariance, split == unsplit, pure-Python brute force, and the
chunked-prefill block arithmetic printed on the Inference Engineering Day 12
page); ``tests/test_oracle_mutants.py`` plants plausible mistakes here and
checks that a pin catches each one.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "kv_head_of",
    "heads_of_kv_head",
    "gather_sequence_kv",
    "attend",
    "merge_partitions",
    "paged_attention_decode",
    "paged_attention_decode_split",
    "paged_attention_prefill",
    "split_reduce",
    "kv_cache_append",
    "fp32_scale",
    "quantize_rows_q8",
    "dequantize_pool_q8",
    "kv_cache_append_q8",
]


def fp32_scale(scale: float) -> float:
    """The softmax scale exactly as an fp32 kernel argument carries it."""
    return float(np.float64(np.float32(scale)))


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head serving query head ``h``: contiguous groups of Hq/Hkv heads."""
    group = num_q_heads // num_kv_heads
    return h // group


def gather_sequence_kv(pool: np.ndarray, table_row: np.ndarray, n: int,
                       block_size: int, kvh: int) -> np.ndarray:
    """Rows 0..n-1 of one sequence's K (or V) for one KV head, as fp64 [n, D].

    Logical position t lives in physical block ``table_row[t // block_size]``
    at offset ``t % block_size`` (nanoserve, "What I built": block allocator
    plus per-sequence block tables).
    """
    t = np.arange(n, dtype=np.int64)
    phys = table_row[t // block_size].astype(np.int64)
    off = t % block_size
    return pool[phys, off, kvh, :].astype(np.float64)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Softmax attention of query rows q [G, D] over K, V [n, D], in fp64.

    Returns (out [G, D], lse [G]) with lse the natural-log log-sum-exp of the
    scaled logits.  n == 0 gives zeros and -inf.
    """
    G, D = q.shape
    n = K.shape[0]
    if n == 0:
        return np.zeros((G, D)), np.full(G, -np.inf)
    s = scale * (q @ K.T)                      # [G, n]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ V) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def heads_of_kv_head(kvh: int, num_q_heads: int, num_kv_heads: int):
    """Query heads served by KV head ``kvh`` (inverse of ``kv_head_of``)."""
    return [h for h in range(num_q_heads)
            if kv_head_of(h, num_q_heads, num_kv_heads) == kvh]


def paged_attention_decode(q, k_pool, v_pool, block_tables, context_lens,
                           scale, return_lse: bool = False, seqs=None):
    """Single-token decode over the paged cache (plain definition, fp64).

    q [B, Hq, D] fp16; pools [NB, bs, Hkv, D] fp16; block_tables [B, maxb]
    int32; context_lens [B] int32.  Returns out [B, Hq, D] fp64 (and lse
    [B, Hq] when asked).  ``seqs`` restricts the work to some sequences; the
    rows of the others stay zero / -inf.  One gather per (sequence, KV head)
    serves the whole query group.
    """
    B, Hq, D = q.shape
    _, bs, Hkv, _ = k_pool.shape
    sc = fp32_scale(scale)
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in (range(B) if seqs is None else seqs):
        n = int(context_lens[b])
        for kvh in range(Hkv):
            heads = heads_of_kv_head(kvh, Hq, Hkv)
            K = gather_sequence_kv(k_pool, block_tables[b], n, bs, kvh)
            V = gather_sequence_kv(v_pool, block_tables[b], n, bs, kvh)
            o, ls = attend(q[b, heads].astype(np.float64), K, V, sc)
            out[b, heads] = o
            lse[b, heads] = ls
    return (out, lse) if return_lse else out


def paged_attention_prefill(q, k_pool, v_pool, block_tables, context_lens, query_start,
                            scale, return_lse: bool = False, seqs=None):
    """Chunked-prefill attention over the paged cache (plain definition, fp64).

    q [total_q, Hq, D] fp16, rows query_start[b] .. query_start[b+1]-1 being
    sequence b's chunk of n_b tokens; context_lens[b] counts the cached
    positions including the chunk.  Row i of the chunk is at position
    p = ctx_b - n_b + i and attends to positions 0..p (a row with p < 0, which
    only a chunk longer than its context has, attends to nothing: zeros,
    lse -inf).  Returns out [total_q, Hq, D] fp64 (and lse [total_q, Hq]).
    ``seqs`` restricts the work to some sequences.
    """
    T, Hq, D = q.shape
    _, bs, Hkv, _ = k_pool.shape
    sc = fp32_scale(scale)
    out = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -np.inf)
    B = len(context_lens)
    for b in (range(B) if seqs is None else seqs):
        r0, r1 = int(query_start[b]), int(query_start[b + 1])
        n, ctx = r1 - r0, int(context_lens[b])
        for kvh in range(Hkv):
            heads = heads_of_kv_head(kvh, Hq, Hkv)
            K = gather_sequence_kv(k_pool, block_tables[b], ctx, bs, kvh)
            V = gather_sequence_kv(v_pool, block_tables[b], ctx, bs, kvh)
            for i in range(n):
                pos = ctx - n + i
                if pos < 0:
                    continue
                o, ls = attend(q[r0 + i, heads].astype(np.float64), K[:pos + 1], V[:pos + 1], sc)
                out[r0 + i, heads] = o
                lse[r0 + i, heads] = ls
    return (out, lse) if return_lse else out


def paged_attention_decode_split(q, k_pool, v_pool, block_tables, context_lens,
                                 scale, partition_size: int,
                                 max_partitions: int):
    """Split-context pass: per partition p of ``partition_size`` logical
    positions, the normalised partial output and its log-sum-exp.

    Returns partial_out [B, Hq, P_max, D] and partial_lse [B, Hq, P_max]
    (fp64).  A partition that starts at or past ctx is empty: lse = -inf and
    a zero output.
    """
    B, Hq, D = q.shape
    _, bs, Hkv, _ = k_pool.shape
    sc = fp32_scale(scale)
    po = np.zeros((B, Hq, max_partitions, D))
    pl = np.full((B, Hq, max_partitions), -np.inf)
    for b in range(B):
        n = int(context_lens[b])
        for kvh in range(Hkv):
            K = gather_sequence_kv(k_pool, block_tables[b], n, bs, kvh)
            V = gather_sequence_kv(v_pool, block_tables[b], n, bs, kvh)
            heads = heads_of_kv_head(kvh, Hq, Hkv)
            qg = q[b, heads].astype(np.float64)
            for p in range(max_partitions):
                lo, hi = p * partition_size, min((p + 1) * partition_size, n)
                if lo >= hi:
                    continue
                o, ls = attend(qg, K[lo:hi], V[lo:hi], sc)
                po[b, heads, p] = o
                pl[b, heads, p] = ls
    return po, pl


def merge_partitions(outs: np.ndarray, lses: np.ndarray):
    """LSE-weighted merge of partial results for one query head.

    outs [P, D], lses [P] (natural log; -inf marks an empty partition).
    LSE = log sum_p exp(lse_p); out = sum_p exp(lse_p - LSE) * out_p.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    if lses.size == 0 or np.all(np.isneginf(lses)):
        return np.zeros(outs.shape[-1]), -np.inf
    mx = lses[np.isfinite(lses)].max()
    w = np.where(np.isneginf(lses), 0.0, np.exp(lses - mx))
    total = w.sum()
    L = mx + np.log(total)
    out = (w[:, None] * np.where(np.isneginf(lses)[:, None], 0.0, outs)).sum(0) / total
    return out, L


def split_reduce(partial_out, partial_lse, context_lens, partition_size: int):
    """Merge the ceil(ctx/partition_size) valid partitions of every
    (sequence, query head).  Returns out [B, Hq, D] and lse [B, Hq] (fp64)."""
    B, Hq, Pm, D = partial_out.shape
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(context_lens[b])
        used = min(Pm, -(-n // partition_size))
        for h in range(Hq):
            out[b, h], lse[b, h] = merge_partitions(partial_out[b, h, :used],
                                                    partial_lse[b, h, :used])
    return out, lse


def kv_cache_append(k_pool, v_pool, k_new, v_new, slot_mapping):
    """Write each new token's K/V rows into its slot; returns new pools.

    k_new, v_new [N, Hkv, D]; slot_mapping [N] int64 with
    slot = physical_block * block_size + offset.  A slot that names no row of
    the pool (slot < 0, or slot >= num_blocks * block_size) is skipped: the
    reading of the Inference Engineering Day 11 post's per-step cache write
    taken here (its addressing is not given on the pages).  The inputs are not
    modified.
    """
    kp = k_pool.copy()
    vp = v_pool.copy()
    nb, bs = kp.shape[0], kp.shape[1]
    flat_k = kp.reshape(nb * bs, *kp.shape[2:])
    flat_v = vp.reshape(nb * bs, *vp.shape[2:])
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = (slots >= 0) & (slots < nb * bs)
    flat_k[slots[keep]] = k_new[keep]
    flat_v[slots[keep]] = v_new[keep]
    return kp, vp


# ---- 8-bit cache ------------------------------------------------------------

def quantize_rows_q8(x16: np.ndarray):
    """int8 codes and fp32 scales of each length-D row of fp16 ``x16`` (last
    axis), with the decisions taken in fp32 as the format defines them."""
    x = np.asarray(x16).astype(np.float32)
    amax = np.max(np.abs(x), axis=-1)
    nz = amax > 0
    inv = np.zeros_like(amax)
    inv[nz] = np.float32(127.0) / amax[nz]
    codes = np.rint(x * inv[..., None])
    codes = np.clip(codes, -127, 127).astype(np.int8)
    scales = (amax / np.float32(127.0)).astype(np.float32)
    return codes, scales


def dequantize_pool_q8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Values code * scale of an 8-bit pool [NB, bs, Hkv, D] (scales
    [NB, bs, Hkv]) in fp64 -- the pool the attention oracles then read."""
    return codes.astype(np.float64) * scales.astype(np.float64)[..., None]


def kv_cache_append_q8(k_codes, v_codes, k_scales, v_scales, k_new, v_new, slot_mapping):
    """Quantise each new token's K and V rows and write codes and scales to
    its slot (copies returned; a negative slot is skipped)."""
    kc, vc = k_codes.copy(), v_codes.copy()
    ks, vs = k_scales.copy(), v_scales.copy()
    nb, bs = kc.shape[:2]
    qk, sk = quantize_rows_q8(k_new)
    qv, sv = quantize_rows_q8(v_new)
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0 or slot >= nb * bs:
            continue
        blk, off = int(slot) // bs, int(slot) % bs
        kc[blk, off], vc[blk, off] = qk[i], qv[i]
        ks[blk, off], vs[blk, off] = sk[i], sv[i]
    return kc, vc, ks, vs
