"""Host block allocator: the reference model pinned by the pages' worked
example and by invariants; the library's C++ allocator (through the C ABI)
equal to the model on seeded random operation sequences.  No GPU needed."""
import json
import os

import numpy as np
import pytest

import paged_kv_decode_cache_amd as pkv
from oracle import paged_ref as ref
from oracle.block_alloc_ref import BlockAllocatorRef, NoSpace

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- pins of the reference model --------------------------------------------

def pin_model_chunked_prefill_golden(model_cls=BlockAllocatorRef):
    """Inference Engineering, Day 12: 8-token chunks into 4-token blocks
    occupy 2 blocks after the first pass and 4 after the second."""
    with open(os.path.join(GOLDEN, "chunked_prefill_blocks.json")) as f:
        g = json.load(f)
    m = model_cls(16, g["block_size"], 2, 8)
    for want in g["blocks_occupied_after_pass"]:
        m.prefill_batch([0], [g["chunk_tokens"]], 8)
        assert 16 - len(m.free) == want
        assert len(m.tables[0]) == want


def _check_invariants(m, num_blocks):
    held = [b for t in m.tables for b in t]
    assert len(held) == len(set(held)), "a block is held twice"
    assert not set(held) & set(m.free), "a held block is also free"
    assert len(held) + len(m.free) == num_blocks, "blocks lost or duplicated"
    for s, t in enumerate(m.tables):
        waste = len(t) * m.block_size - m.lens[s]
        assert 0 <= waste < m.block_size, f"sequence {s} wastes {waste} slots"


def pin_model_invariants_under_churn(model_cls=BlockAllocatorRef):
    """Random appends, frees and batches: no block is lost or shared, and
    every sequence wastes less than one block (nanoserve, "What I built")."""
    rng = np.random.default_rng(500)
    NB, bs, S = 64, 16, 8
    m = model_cls(NB, bs, S, 16)
    for _ in range(400):
        op = rng.integers(4)
        s = int(rng.integers(S))
        try:
            if op == 0:
                slots = m.append_slots(s, int(rng.integers(0, 40)))
                # each slot decomposes to (its table's block, its offset)
                first = m.lens[s] - len(slots)
                for i, sl in enumerate(slots):
                    p = first + i
                    assert sl // bs == m.tables[s][p // bs] and sl % bs == p % bs
            elif op == 1:
                m.free_seq(s)
            elif op == 2:
                seqs = list(rng.choice(S, size=int(rng.integers(1, S)), replace=False))
                m.decode_batch([int(x) for x in seqs], 16)
            else:
                seqs = [int(x) for x in rng.choice(S, size=3, replace=False)]
                m.prefill_batch(seqs, [int(x) for x in rng.integers(0, 30, 3)], 16)
        except (NoSpace, ValueError):
            pass
        _check_invariants(m, NB)


def pin_model_queue_order(model_cls=BlockAllocatorRef):
    """The free blocks form a queue: fresh blocks come out in order, and a
    freed sequence's blocks come back after those already waiting."""
    m = model_cls(6, 4, 3, 6)
    m.append_slots(0, 8)                 # takes 0, 1
    m.append_slots(1, 4)                 # takes 2
    m.free_seq(0)                        # queue: 3, 4, 5, 0, 1
    m.append_slots(2, 20)                # takes 3, 4, 5, 0, 1
    assert m.tables[2] == [3, 4, 5, 0, 1]


def pin_model_all_or_nothing(model_cls=BlockAllocatorRef):
    """A request that does not fit changes nothing."""
    m = model_cls(3, 4, 3, 4)
    m.append_slots(0, 4)                 # one full block held, two free
    state = lambda: (list(m.free), [list(t) for t in m.tables], list(m.lens))
    snap = state()
    for call in (lambda: m.prefill_batch([1, 2], [4, 5], 4),   # needs 3 blocks
                 lambda: m.decode_batch([0, 1, 2], 4),         # needs 3 blocks
                 lambda: m.append_slots(2, 13),                # needs 4 blocks
                 lambda: m.append_slots(0, 13)):               # past 4 blocks per table
        with pytest.raises(NoSpace):
            call()
        assert state() == snap


MODEL_PINS = (pin_model_chunked_prefill_golden, pin_model_invariants_under_churn,
              pin_model_queue_order, pin_model_all_or_nothing)


@pytest.mark.parametrize("pin", MODEL_PINS, ids=[p.__name__ for p in MODEL_PINS])
def test_reference_model_pins(pin):
    pin()


class _Lifo(BlockAllocatorRef):
    def append_slots(self, seq, n):
        want = self._blocks_for(self.lens[seq] + n)
        if want > self.max_blocks_per_seq or want - len(self.tables[seq]) > len(self.free):
            raise NoSpace("full")
        while len(self.tables[seq]) < want:
            self.tables[seq].append(self.free.pop())          # stack, not queue
        first = self.lens[seq]
        self.lens[seq] += n
        return [self.slot_of(seq, p) for p in range(first, first + n)]


class _OneBlockTooMany(BlockAllocatorRef):
    def _blocks_for(self, n_tokens):
        return n_tokens // self.block_size + 1                # a whole spare block


class _NoRequeue(BlockAllocatorRef):
    def free_seq(self, seq):
        self.tables[seq] = []
        self.lens[seq] = 0


@pytest.mark.parametrize("mutant", [_Lifo, _OneBlockTooMany, _NoRequeue],
                         ids=["lifo", "spare_block", "no_requeue"])
def test_a_model_pin_catches_mutant(mutant):
    caught = 0
    for pin in MODEL_PINS:
        try:
            pin(mutant)
        except (AssertionError, NoSpace, ValueError, IndexError):
            caught += 1
    assert caught, f"no pin catches {mutant.__name__}"


# ---- the library's allocator against the model ------------------------------

def _same_state(a, m, S, width):
    assert a.num_free == len(m.free)
    for s in range(S):
        assert a.context_len(s) == m.lens[s]
        assert list(a.block_table(s, width)) == m.block_table(s, width)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_library_allocator_equals_model(seed):
    rng = np.random.default_rng(510 + seed)
    NB, bs, S, W = int(rng.integers(8, 80)), int(rng.choice([1, 4, 16])), 6, 12
    a = pkv.BlockAllocator(NB, bs, S, W)
    m = BlockAllocatorRef(NB, bs, S, W)
    for _ in range(300):
        op = int(rng.integers(5))
        s = int(rng.integers(S))
        outcome = []
        for side in ("lib", "model"):
            try:
                if op == 0:
                    n = int(rng.integers(0, 3 * bs + 2)) if side == "lib" else n
                    r = a.append_slots(s, n) if side == "lib" else m.append_slots(s, n)
                    outcome.append(("ok", list(map(int, r))))
                elif op == 1:
                    (a.free(s) if side == "lib" else m.free_seq(s))
                    outcome.append(("ok",))
                elif op == 2:
                    if side == "lib":
                        seqs = [int(x) for x in rng.choice(S, size=int(rng.integers(0, S + 1)),
                                                           replace=False)]
                    r = a.decode_batch(seqs, W) if side == "lib" else m.decode_batch(seqs, W)
                    outcome.append(("ok", [list(map(int, np.ravel(x))) for x in r]))
                elif op == 3:
                    if side == "lib":
                        seqs = [int(x) for x in rng.choice(S, size=int(rng.integers(0, 4)),
                                                           replace=False)]
                        chunks = [int(x) for x in rng.integers(0, 2 * bs + 3, len(seqs))]
                    r = (a.prefill_batch(seqs, chunks, W) if side == "lib"
                         else m.prefill_batch(seqs, chunks, W))
                    outcome.append(("ok", [list(map(int, np.ravel(x))) for x in r]))
                else:
                    if side == "lib":
                        seqs = [s, s]
                    r = a.decode_batch(seqs, W) if side == "lib" else m.decode_batch(seqs, W)
                    outcome.append(("ok",))
            except (pkv.NoSpaceError, NoSpace):
                outcome.append(("nospace",))
            except ValueError:
                outcome.append(("invalid",))
        assert outcome[0] == outcome[1], (op, outcome)
        _same_state(a, m, S, W)


def test_library_allocator_rejects_bad_arguments():
    with pytest.raises(ValueError):
        pkv.BlockAllocator(0, 16, 4, 4)
    a = pkv.BlockAllocator(8, 16, 2, 4)
    with pytest.raises(ValueError):
        a.append_slots(2, 1)                      # sequence id out of range
    with pytest.raises(ValueError):
        a.append_slots(0, -1)
    with pytest.raises(ValueError):
        a.decode_batch([0, 0], 4)                 # repeated id
    a.append_slots(0, 40)                         # 3 blocks
    with pytest.raises(ValueError):
        a.block_table(0, 2)                       # width below the table
    with pytest.raises(ValueError):
        a.decode_batch([0], 2)
    with pytest.raises(pkv.NoSpaceError):
        a.append_slots(0, 100)                    # past max_blocks_per_seq
    assert a.context_len(0) == 40 and a.num_free == 5
    lib = pkv.load_library()
    assert lib.pkv_allocator_num_free(None) == pkv.PKV_ERR_INVALID_ARG
    assert lib.pkv_allocator_append_slots(None, 0, 1, None) == pkv.PKV_ERR_INVALID_ARG
    assert pkv.status_string(pkv.PKV_ERR_NO_SPACE).startswith("no space")


def test_allocator_slots_drive_the_oracle_append():
    """Slots and tables from the library's allocator, fed to the oracle's
    append and gather, give back every sequence's token history."""
    rng = np.random.default_rng(520)
    NB, bs, Hkv, D, S = 40, 16, 2, 8, 5
    a = pkv.BlockAllocator(NB, bs, S, 8)
    kp = np.full((NB, bs, Hkv, D), np.nan, dtype=np.float16)
    vp = kp.copy()
    hist = [np.zeros((0, Hkv, D), np.float16) for _ in range(S)]
    for step in range(25):
        if step % 7 == 6:
            s = int(rng.integers(S))
            a.free(s)
            hist[s] = hist[s][:0]
        seqs = [int(x) for x in rng.choice(S, size=3, replace=False)]
        chunks = [int(x) for x in rng.integers(1, 20, 3)]
        try:
            qs, slots, tables, lens = a.prefill_batch(seqs, chunks, 8)
        except pkv.NoSpaceError:
            continue
        kn = rng.standard_normal((int(qs[-1]), Hkv, D)).astype(np.float16)
        kp, vp = ref.kv_cache_append(kp, vp, kn, kn, slots)
        for b, s in enumerate(seqs):
            hist[s] = np.concatenate([hist[s], kn[qs[b]:qs[b + 1]]])
        for s in range(S):
            n = a.context_len(s)
            assert n == len(hist[s])
            row = a.block_table(s, 8)
            for kvh in range(Hkv):
                got = ref.gather_sequence_kv(kp, row, n, bs, kvh)
                assert np.array_equal(got, hist[s][:, kvh].astype(np.float64))
