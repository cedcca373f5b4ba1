"""Pins of the block-manager oracle (CPU): block counts against the pages'
examples, slots against the skill page's address rule, the first-free
allocation order, reference counting over forks, copy-on-write of a shared
partial block, refusal without side effects, pending-copy locking, and the
bookkeeping invariants over random operation scripts. Planted mistakes at
the end must each fail a pin."""

import json
import os
import random

import numpy as np
import pytest

import oracle
import oracle.block_manager as obm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_block_counts_match_the_pages_examples():
    ex = json.load(open(os.path.join(GOLDEN, "block_counts.json")))["examples"]
    for e in ex:
        bm = oracle.BlockManager(4096, e["block_size"])
        bm.add_sequence(0)
        st, slots = bm.append(0, e["tokens"])
        assert st == 0 and len(bm.tables[0]) == e["blocks"]


def test_slots_follow_the_address_rule():
    bm = oracle.BlockManager(64, 16)
    for s in range(3):
        bm.add_sequence(s)
    got = {s: [] for s in range(3)}
    for step, (s, n) in enumerate([(0, 20), (1, 5), (0, 13), (2, 40), (1, 30), (0, 1)]):
        st, slots = bm.append(s, n)
        assert st == 0
        got[s] += slots
    for s in range(3):
        st, rows, lens = bm.block_table([s], 8)
        table = np.array(rows, dtype=np.int32)
        want = [oracle.slot_of(table, 0, p, 16) for p in range(lens[0])]
        assert got[s] == want


def test_first_sequence_on_a_fresh_pool_gets_the_identity_slots():
    """Skill page section 3.3: with the identity table the first sequence's
    prefill slots are 0..kv_len-1 and its decode slot is kv_len (bs 128)."""
    bm = oracle.BlockManager(32, 128)
    bm.add_sequence(0)
    assert bm.append(0, 512)[1] == list(range(512))
    bm2 = oracle.BlockManager(32, 128)
    bm2.add_sequence(0)
    bm2.append(0, 522)
    assert bm2.append(0, 1)[1] == [522]


def test_first_free_block_is_taken():
    bm = oracle.BlockManager(8, 4)
    for s in "ABC":
        bm.add_sequence(s)
    bm.append("A", 12)
    bm.append("B", 8)
    assert bm.tables["A"] == [0, 1, 2] and bm.tables["B"] == [3, 4]
    bm.free_sequence("A")
    bm.append("C", 16)
    assert bm.tables["C"] == [0, 1, 2, 5]
    assert bm.num_free() == 2


def test_fork_shares_blocks_and_counts_references():
    bm = oracle.BlockManager(8, 4)
    bm.add_sequence(1)
    bm.append(1, 8)
    assert bm.fork(1, 2) == 0
    assert bm.tables[2] == [0, 1] and bm.ref[:2] == [2, 2]
    free_before = bm.num_free()
    bm.free_sequence(1)
    assert bm.ref[:2] == [1, 1] and bm.num_free() == free_before
    bm.free_sequence(2)
    assert bm.num_free() == 8


def test_copy_on_write_of_a_shared_partial_block():
    bm = oracle.BlockManager(8, 4)
    bm.add_sequence(1)
    bm.append(1, 6)                 # blocks [0, 1], block 1 half full
    bm.fork(1, 2)
    st, slots = bm.append(2, 1)     # child writes position 6 -> into a copy of block 1
    assert st == 0
    assert bm.tables[1] == [0, 1] and bm.tables[2] == [0, 2]
    assert slots == [2 * 4 + 2]
    assert bm.ref[:3] == [2, 1, 1]
    assert bm.take_copies() == [(1, 2)]
    assert bm.take_copies() == []


def test_no_copy_when_the_shared_block_is_full():
    bm = oracle.BlockManager(8, 4)
    bm.add_sequence(1)
    bm.append(1, 8)
    bm.fork(1, 2)
    st, slots = bm.append(2, 1)
    assert st == 0 and bm.tables[2] == [0, 1, 2] and slots == [8]
    assert bm.take_copies() == []


def test_out_of_blocks_changes_nothing():
    bm = oracle.BlockManager(4, 4)
    bm.add_sequence(1)
    bm.append(1, 10)
    snapshot = (list(bm.ref), list(bm.tables[1]), bm.lens[1])
    st, slots = bm.append(1, 7)     # needs 2 more blocks, 1 free
    assert st == obm.ERR_NO_BLOCKS and slots == []
    assert (list(bm.ref), list(bm.tables[1]), bm.lens[1]) == snapshot


def test_unknown_and_duplicate_sequences_are_refused():
    bm = oracle.BlockManager(4, 4)
    assert bm.append(9, 1)[0] == obm.ERR_SHAPE
    assert bm.free_sequence(9) == obm.ERR_SHAPE
    bm.add_sequence(1)
    assert bm.add_sequence(1) == obm.ERR_SHAPE
    assert bm.fork(1, 1) == obm.ERR_SHAPE and bm.fork(7, 2) == obm.ERR_SHAPE
    assert bm.block_table([1, 9], 4)[0] == obm.ERR_SHAPE


def test_blocks_of_pending_copies_are_not_reused():
    bm = oracle.BlockManager(4, 4)
    bm.add_sequence(1)
    bm.append(1, 2)                 # block 0
    bm.fork(1, 2)
    bm.append(2, 1)                 # copy 0 -> 1; child on block 1
    bm.free_sequence(1)
    bm.free_sequence(2)             # blocks 0 and 1 free but named by the pending pair
    bm.add_sequence(3)
    assert bm.append(3, 8)[0] == 0 and bm.tables[3] == [2, 3]
    assert bm.append(3, 1)[0] == obm.ERR_NO_BLOCKS
    bm.take_copies()
    assert bm.append(3, 1)[0] == 0 and bm.tables[3] == [2, 3, 0]


def test_copy_from_a_pending_destination_is_refused():
    bm = oracle.BlockManager(8, 4)
    bm.add_sequence(1)
    bm.append(1, 2)
    bm.fork(1, 2)
    bm.append(2, 1)                 # child now on block 1, copy (0, 1) pending
    bm.fork(2, 3)
    assert bm.append(3, 1)[0] == obm.ERR_PENDING_COPY
    assert bm.take_copies() == [(0, 1)]
    assert bm.append(3, 1)[0] == 0 and bm.take_copies() == [(1, 2)]


def test_copy_blocks_applies_pairs_in_order():
    pool = np.arange(5 * 3).reshape(5, 3)
    out = oracle.copy_blocks(pool, [(0, 4), (2, 1)])
    assert out[4].tolist() == pool[0].tolist() and out[1].tolist() == pool[2].tolist()
    assert out[0].tolist() == pool[0].tolist() and out[3].tolist() == pool[3].tolist()


def check_invariants(bm):
    count = [0] * bm.num_blocks
    for s, t in bm.tables.items():
        assert len(t) == -(-bm.lens[s] // bm.block_size)
        for b in t:
            count[b] += 1
    assert count == bm.ref
    assert bm.num_free() == sum(1 for r in bm.ref if r == 0)
    srcs = [p[0] for p in bm.pending]
    dsts = [p[1] for p in bm.pending]
    assert len(set(dsts)) == len(dsts) and not set(srcs) & set(dsts)


def random_script(seed, n_ops=400, num_blocks=48, bs=4):
    rng = random.Random(seed)
    ops, live, nxt = [], [], 0
    for _ in range(n_ops):
        r = rng.random()
        if r < 0.15 or not live:
            ops.append(("add", nxt)); live.append(nxt); nxt += 1
        elif r < 0.25:
            ops.append(("fork", rng.choice(live), nxt)); live.append(nxt); nxt += 1
        elif r < 0.35:
            s = rng.choice(live); live.remove(s); ops.append(("free", s))
        elif r < 0.42:
            ops.append(("take",))
        else:
            ops.append(("append", rng.choice(live), rng.choice([1, 1, 1, 2, 3, 5, 9])))
    return num_blocks, bs, ops


def run_script(bm, ops):
    """Apply ops; return every observable output (for the invariants here and
    for the library parity test)."""
    trace = []
    for op in ops:
        if op[0] == "add":
            trace.append(bm.add_sequence(op[1]))
        elif op[0] == "fork":
            trace.append(bm.fork(op[1], op[2]))
        elif op[0] == "free":
            trace.append(bm.free_sequence(op[1]))
        elif op[0] == "take":
            trace.append(tuple(bm.take_copies()))
        else:
            trace.append(bm.append(op[1], op[2]))
        trace.append(bm.num_free())
    return trace


@pytest.mark.parametrize("seed", range(6))
def test_invariants_hold_over_random_scripts(seed):
    nb, bs, ops = random_script(seed)
    bm = oracle.BlockManager(nb, bs)
    for op in ops:
        run_script(bm, [op])
        check_invariants(bm)


# ---- planted mistakes ------------------------------------------------------

def _last_free(self):
    for b in reversed(range(self.num_blocks)):
        if self.ref[b] == 0 and b not in self.locked:
            self.ref[b] = 1
            return b
    raise AssertionError


def _release_never(self, b):
    pass


PINS = [test_block_counts_match_the_pages_examples, test_slots_follow_the_address_rule,
        test_first_sequence_on_a_fresh_pool_gets_the_identity_slots, test_first_free_block_is_taken,
        test_fork_shares_blocks_and_counts_references, test_copy_on_write_of_a_shared_partial_block,
        test_no_copy_when_the_shared_block_is_full, test_out_of_blocks_changes_nothing,
        test_blocks_of_pending_copies_are_not_reused, test_copy_from_a_pending_destination_is_refused]


def _append_no_cow(self, seq, n):
    saved = self.ref
    self.ref = [min(r, 1) for r in saved]     # every block looks unshared
    try:
        return _REAL_APPEND(self, seq, n)
    finally:
        self.ref = [max(a, b) for a, b in zip(saved, self.ref)]


def _append_extra_block(self, seq, n):
    st, slots = _REAL_APPEND(self, seq, n)
    if st == 0 and n and self.lens[seq] % self.block_size == 0 and self._num_allocatable():
        self.tables[seq].append(self._take_free())
    return st, slots


_REAL_APPEND = obm.BlockManager.append


@pytest.mark.parametrize("name,attr,fake", [
    ("last free block first", "_take_free", _last_free),
    ("release never frees", "_release", _release_never),
    ("no copy-on-write", "append", _append_no_cow),
    ("one block too many on an exact fill", "append", _append_extra_block),
])
def test_a_pin_catches_the_planted_mistake(monkeypatch, name, attr, fake):
    monkeypatch.setattr(obm.BlockManager, attr, fake)
    caught = 0
    for t in PINS:
        try:
            t()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught: {name}"
