"""CPU pins of the block-manager oracle (oracle.blocks) against what P3 §3-§4
fix and against reference-counting invariants checked by brute force.

Every pin is a plain function taking the manager class, so that the mutation
test at the bottom can re-run the pins against managers with planted
mistakes.
"""
import copy
import json
import os
import random

import pytest

import oracle.blocks as OB
import oracle.paged as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# invariants, checked from scratch after every operation
# ---------------------------------------------------------------------------

def check_invariants(bm):
    """Reference counts equal the number of table entries naming each block;
    the free queue holds exactly the unreferenced blocks, once each; the
    allocated count is their complement."""
    pool = bm.pool
    count = [0] * pool.total
    for table in bm.tables.values():
        for b in table:
            count[b] += 1
    assert count == pool.ref, "reference counts differ from table multiplicities"
    free = list(pool.free_queue)
    assert len(free) == len(set(free)), "a block is queued twice"
    assert sorted(free) == [b for b in range(pool.total) if count[b] == 0], \
        "free queue differs from the set of unreferenced blocks"
    assert pool.allocated == pool.total - len(free)


class ContentModel:
    """Shadow contents of the pool: what each slot holds, written only through
    the slots and copies the manager hands out (the way the GPU pool is)."""

    def __init__(self, num_blocks, block_size):
        self.B = block_size
        self.slots = [None] * (num_blocks * block_size)
        self.expected = {}          # request -> list of token labels it must read back

    def copy_block(self, src, dst):
        B = self.B
        self.slots[dst * B:(dst + 1) * B] = self.slots[src * B:(src + 1) * B]

    def write(self, slot, label):
        self.slots[slot] = label

    def check(self, bm):
        for rid, labels in self.expected.items():
            table = bm.tables[rid]
            for t, lab in enumerate(labels):
                slot = P.slot_of(table, t, self.B)
                assert slot >= 0 and self.slots[slot] == lab, \
                    f"request {rid} reads {self.slots[slot] if slot >= 0 else None} at token {t}, wrote {lab}"


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def test_pin_bm_pages_scenario(cls=OB.BlockManager):
    """P3 §3's closing example (fixture with citation)."""
    g = _golden("p3_manager_scenario.json")
    bm = cls(g["num_blocks"], g["block_size"])
    assert bm.allocate_for_request(1, g["prompt_tokens"]) == g["prompt_blocks"]
    slot, new_block, cp = bm.append_slot(1, g["append_position"])
    assert (new_block is not None) == g["append_allocates"] and cp is None
    a = bm.table(1)
    assert slot == a[g["append_position"] // g["block_size"]] * g["block_size"] + \
        g["append_position"] % g["block_size"]
    bm.share_prefix_blocks(1, 2, g["shared_tokens"])
    assert bm.table(2) == a[:g["shared_blocks"]]
    for b in a[:g["shared_blocks"]]:
        assert bm.pool.ref[b] == 2
    check_invariants(bm)
    bm.free_request(1)
    # the shared blocks survive the first holder's release
    assert all(bm.pool.ref[b] == 1 for b in a[:g["shared_blocks"]])
    assert all(b not in bm.free_ids() for b in a[:g["shared_blocks"]])
    bm.free_request(2)
    assert bm.num_free() == g["free_after_all"] and bm.pool.allocated == 0
    check_invariants(bm)


def test_pin_bm_fifo_order(cls=OB.BlockManager):
    """P3 §3: allocation takes the front of the free queue, release appends at
    the back."""
    bm = cls(8, 4)
    bm.allocate_for_request(10, 12)          # 3 blocks
    assert bm.table(10) == [0, 1, 2]
    bm.allocate_for_request(11, 1)
    assert bm.table(11) == [3]
    bm.free_request(10)
    assert bm.free_ids() == [4, 5, 6, 7, 0, 1, 2]
    bm.allocate_for_request(12, 5)
    assert bm.table(12) == [4, 5]


def test_pin_bm_all_or_nothing(cls=OB.BlockManager):
    """P3 §3: a prompt that does not fit leaves the pool untouched."""
    bm = cls(5, 16)
    bm.allocate_for_request(1, 48)           # 3 blocks, 2 left
    before = copy.deepcopy((bm.tables, list(bm.pool.free_queue), bm.pool.ref, bm.pool.allocated))
    with pytest.raises(OB.BlockError) as e:
        bm.allocate_for_request(2, 33)       # needs 3
    assert e.value.kind == "no_blocks"
    after = (bm.tables, list(bm.pool.free_queue), bm.pool.ref, bm.pool.allocated)
    assert after == before


def test_pin_bm_append_boundaries(cls=OB.BlockManager):
    """B2: token p lives in logical block p // B; the block is allocated when
    p opens it, and only then."""
    bm = cls(16, 4)
    bm.allocate_for_request(1, 5)            # tokens 0..4 -> 2 blocks
    assert bm.append_slot(1, 5)[1] is None   # inside block 1
    assert bm.append_slot(1, 7)[1] is None
    slot, nb, _ = bm.append_slot(1, 8)       # opens block 2
    assert nb is not None and bm.table(1)[2] == nb and slot == nb * 4
    with pytest.raises(OB.BlockError):
        bm.append_slot(1, 16)                # would skip block 3
    bm2 = cls(2, 4)
    bm2.allocate_for_request(1, 8)
    with pytest.raises(OB.BlockError) as e:
        bm2.append_slot(1, 8)
    assert e.value.kind == "no_blocks"


def test_pin_bm_errors(cls=OB.BlockManager):
    bm = cls(4, 16)
    with pytest.raises(OB.BlockError) as e:
        bm.free_request(7)
    assert e.value.kind == "unknown_request"
    bm.allocate_for_request(1, 10)
    with pytest.raises(OB.BlockError):
        bm.allocate_for_request(1, 10)       # id in use
    with pytest.raises(OB.BlockError):
        bm.share_prefix_blocks(1, 2, 17)     # source has 1 block, 2 needed
    with pytest.raises(OB.BlockError):
        bm.pool.free(3)                      # never allocated
    bm.free_request(1)
    with pytest.raises(OB.BlockError):
        bm.free_request(1)


def _random_session(cls, seed, num_blocks=24, block_size=4, steps=400):
    """Random allocate / append / share / fork / free traffic with the
    invariants and the shadow contents checked after every step."""
    rng = random.Random(seed)
    bm = cls(num_blocks, block_size)
    cm = ContentModel(num_blocks, block_size)
    lens = {}
    next_id = 1
    label = 0
    for _ in range(steps):
        op = rng.random()
        live = sorted(bm.tables)
        state = copy.deepcopy((bm.tables, list(bm.pool.free_queue), bm.pool.ref))
        try:
            if op < 0.25 or not live:
                n = rng.randint(0, 3 * block_size)
                bm.allocate_for_request(next_id, n)
                labs = []
                for t in range(n):
                    label += 1
                    cm.write(P.slot_of(bm.tables[next_id], t, block_size), label)
                    labs.append(label)
                cm.expected[next_id] = labs
                lens[next_id] = n
                next_id += 1
            elif op < 0.65:
                rid = rng.choice(live)
                slot, nb, cp = bm.append_slot(rid, lens[rid])
                if cp is not None:
                    cm.copy_block(*cp)
                label += 1
                cm.write(slot, label)
                cm.expected[rid].append(label)
                lens[rid] += 1
            elif op < 0.8:
                src = rng.choice(live)
                n = rng.randint(0, lens[src])
                bm.share_prefix_blocks(src, next_id, n)
                cm.expected[next_id] = list(cm.expected[src][:n])
                lens[next_id] = n
                next_id += 1
            elif op < 0.85:
                src = rng.choice(live)
                bm.fork(src, next_id)
                cm.expected[next_id] = list(cm.expected[src])
                lens[next_id] = lens[src]
                next_id += 1
            else:
                rid = rng.choice(live)
                bm.free_request(rid)
                del cm.expected[rid], lens[rid]
        except OB.BlockError as e:
            assert e.kind == "no_blocks"
            assert copy.deepcopy((bm.tables, list(bm.pool.free_queue), bm.pool.ref)) == state, \
                "a refused operation changed the state"
        check_invariants(bm)
        cm.check(bm)
    return bm


def test_pin_bm_random_sessions(cls=OB.BlockManager):
    for seed in range(6):
        _random_session(cls, seed)


def test_pin_bm_copy_on_write(cls=OB.BlockManager):
    """B3: appending into a block another request holds copies it first; the
    other holder keeps the original."""
    bm = cls(8, 4)
    bm.allocate_for_request(1, 6)            # blocks 0, 1 (block 1 half full)
    bm.share_prefix_blocks(1, 2, 6)          # request 2 shares both
    slot, nb, cp = bm.append_slot(2, 6)
    assert cp == (1, nb) and bm.table(2) == [0, nb] and bm.table(1) == [0, 1]
    assert slot == nb * 4 + 2
    assert bm.pool.ref[1] == 1 and bm.pool.ref[0] == 2
    slot1, nb1, cp1 = bm.append_slot(1, 6)   # sole holder now: in place
    assert cp1 is None and nb1 is None and slot1 == 1 * 4 + 2


# ---------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin
# ---------------------------------------------------------------------------

class _SaturatingPool(OB.BlockPool):
    """The listing taken literally: free saturates at zero instead of failing,
    and allocate does not record the count on the pooled block."""

    def allocate(self):
        if not self.free_queue:
            return None
        b = self.free_queue.popleft()
        self.allocated += 1
        return b

    def free(self, b):
        self.ref[b] = max(self.ref[b] - 1, 0)
        if self.ref[b] == 0:
            self.free_queue.append(b)
            self.allocated -= 1

    def add_ref(self, b):
        self.ref[b] += 1


class _LifoPool(OB.BlockPool):
    def free(self, b):
        if self.ref[b] <= 0:
            raise OB.BlockError("state", "double free")
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free_queue.appendleft(b)
            self.allocated -= 1


def _with_pool(pool_cls):
    class M(OB.BlockManager):
        def __init__(self, n, b):
            super().__init__(n, b)
            self.pool = pool_cls(n)
    return M


class _NoCopyOnWrite(OB.BlockManager):
    def append_slot(self, rid, position):
        table = self._table(rid)
        B = self.block_size
        logical, offset = position // B, position % B
        if logical > len(table):
            raise OB.BlockError("state", "skip")
        nb = None
        if logical == len(table):
            b = self.pool.allocate()
            if b is None:
                raise OB.BlockError("no_blocks", "none")
            table.append(b)
            nb = b
        return table[logical] * B + offset, nb, None


class _NoRollback(OB.BlockManager):
    def allocate_for_request(self, rid, num_tokens):
        need = OB.num_required_blocks(num_tokens, self.block_size)
        table = []
        for _ in range(need):
            b = self.pool.allocate()
            if b is None:
                self.tables[rid] = table
                raise OB.BlockError("no_blocks", "partial")
            table.append(b)
        self.tables[rid] = table
        return need


class _AllocateAtEveryBoundary(OB.BlockManager):
    """The listing's append rule: a new block whenever the position is a
    multiple of B, whether or not the table already has it."""

    def append_slot(self, rid, position):
        table = self._table(rid)
        B = self.block_size
        nb = None
        if position % B == 0:
            b = self.pool.allocate()
            if b is None:
                raise OB.BlockError("no_blocks", "none")
            table.append(b)
            nb = b
        return table[position // B] * B + position % B, nb, None


_PINS = [v for k, v in sorted(globals().items()) if k.startswith("test_pin_bm_")]


@pytest.mark.parametrize("mutant", [_with_pool(_SaturatingPool), _with_pool(_LifoPool),
                                    _NoCopyOnWrite, _NoRollback, _AllocateAtEveryBoundary],
                         ids=["saturating-free", "lifo", "no-copy-on-write", "no-rollback",
                              "allocate-at-every-boundary"])
def test_block_mutants_are_caught(mutant):
    failed = []
    for pin in _PINS:
        try:
            pin(mutant)
        except (Exception, pytest.fail.Exception):      # noqa: BLE001 - any failure counts
            failed.append(pin.__name__)
    assert failed, "no pin caught this planted mistake"
