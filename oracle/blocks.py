"""Plain reference for the host-side KV block manager -- TEST INFRASTRUCTURE ONLY.

Follows the block pool and request manager of P3 §3 (the Rust listing of a
paged KV-cache manager) step by step, with the readings below.  Pure Python,
no speed-ups; see the package docstring for who may use it and for the
source keys.

What P3 §3 describes:
* A pool of ``num_blocks`` physical blocks.  Free blocks wait in a FIFO queue
  (taken from the front, returned to the back); every block carries a
  reference count.
* ``allocate`` takes the front block and gives it one reference;
  ``free`` drops one reference and returns the block to the queue when none
  is left; ``add_ref`` adds one (sharing).  Usage = allocated / total.
* A request's block table lists its physical block ids in logical order;
  ``num_required_blocks`` rounds up.
* ``allocate_for_request`` is all-or-nothing: it fails without side effects
  when the pool lacks the blocks.
* ``append_slot`` gives a decoding request a new block when its newest token
  opens one; with no free block it reports that preemption is needed.
* ``free_request`` drops the references of every block of the request.
* ``share_prefix_blocks`` builds a new request's table from the first
  ceil(shared_len / B) blocks of another request, adding a reference to each
  (P3 §3; P3 §4: a beam-search fork copies block references the same way).

Readings where the listing is silent or at odds with its own comments:
* B1 (reference counts): the listing sets the count on a copy of the popped
  block and saturates at zero on free, so a shared block could return to the
  queue while a holder still uses it; its comments state the intent (a block
  is recycled only when every holder has released it).  Taken: the count
  lives with the block, allocate sets it to 1, add_ref adds 1, free
  subtracts 1 and recycles at 0; freeing or sharing a block whose count is
  already 0 is an error, not a saturation.
* B2 (token positions): 0-based (token 17 is logical block 1, offset 1).  A
  request grows one token at a time: appending position p needs logical
  block p // B; that block is allocated when it is the first block past the
  table (p // B == len(table)); a position further out is an error.
* B3 (writing into a shared block): the pages do not say what happens when a
  request that shares a partly filled block appends into it.  Taken: copy on
  write -- the request drops its reference to the shared block, receives a
  fresh block, and the caller is told to copy the old block's contents into
  it (the block-copy kernel) before writing the new token.  Blocks with one
  holder are written in place.
* B4 (request ids): allocating or sharing into an id that already has a
  table is an error; operations on an unknown id are errors (the listing's
  "Request not found").
"""
from __future__ import annotations

from collections import deque


class BlockError(Exception):
    """A refused operation.  ``kind`` is one of 'no_blocks', 'unknown_request',
    'state', 'invalid'."""

    def __init__(self, kind: str, message: str):
        super().__init__(f"{kind}: {message}")
        self.kind = kind


def num_required_blocks(num_tokens: int, block_size: int) -> int:
    """P3 §3: blocks needed for ``num_tokens`` tokens, rounding up."""
    return (num_tokens + block_size - 1) // block_size


class BlockPool:
    """P3 §3 block pool: FIFO free queue of ids plus a count per block (B1)."""

    def __init__(self, num_blocks: int):
        if num_blocks <= 0:
            raise BlockError("invalid", "num_blocks must be > 0")
        self.total = num_blocks
        self.free_queue = deque(range(num_blocks))
        self.ref = [0] * num_blocks
        self.allocated = 0

    def allocate(self):
        """Front of the queue with one reference, or None when empty."""
        if not self.free_queue:
            return None
        b = self.free_queue.popleft()
        self.ref[b] = 1
        self.allocated += 1
        return b

    def free(self, b: int) -> None:
        """Drop one reference; back of the queue at zero (B1)."""
        if self.ref[b] <= 0:
            raise BlockError("state", f"block {b} is not allocated")
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free_queue.append(b)
            self.allocated -= 1

    def add_ref(self, b: int) -> None:
        if self.ref[b] <= 0:
            raise BlockError("state", f"block {b} is not allocated")
        self.ref[b] += 1

    def usage_ratio(self) -> float:
        return self.allocated / self.total


class BlockManager:
    """P3 §3 request manager over one pool of blocks of ``block_size`` tokens."""

    def __init__(self, num_blocks: int, block_size: int):
        if block_size <= 0:
            raise BlockError("invalid", "block_size must be > 0")
        self.block_size = block_size
        self.pool = BlockPool(num_blocks)
        self.tables: dict[int, list[int]] = {}

    def _table(self, rid: int) -> list[int]:
        if rid not in self.tables:
            raise BlockError("unknown_request", f"request {rid} not found")
        return self.tables[rid]

    def allocate_for_request(self, rid: int, num_tokens: int) -> int:
        """All-or-nothing allocation of the blocks for a prompt of
        ``num_tokens`` tokens; returns the number of blocks."""
        if num_tokens < 0:
            raise BlockError("invalid", "num_tokens must be >= 0")
        if rid in self.tables:
            raise BlockError("state", f"request {rid} already has a table")
        need = num_required_blocks(num_tokens, self.block_size)
        if len(self.pool.free_queue) < need:
            raise BlockError("no_blocks", f"need {need}, available {len(self.pool.free_queue)}")
        table = []
        for _ in range(need):
            table.append(self.pool.allocate())
        self.tables[rid] = table
        return need

    def append_slot(self, rid: int, position: int):
        """Make room for the token at ``position`` (B2, B3).

        Returns ``(slot, new_block, copy)``: the token's slot
        (phys * B + offset), the id of a block allocated by this call (or
        None), and ``(src, dst)`` when the token's block was shared and had to
        be copied first (or None).
        """
        table = self._table(rid)
        B = self.block_size
        if position < 0:
            raise BlockError("invalid", "position must be >= 0")
        logical, offset = position // B, position % B
        if logical > len(table):
            raise BlockError("state", f"position {position} skips past the end of the table")
        new_block, copy = None, None
        if logical == len(table):
            b = self.pool.allocate()
            if b is None:
                raise BlockError("no_blocks", "preemption required: no free blocks")
            table.append(b)
            new_block = b
        else:
            old = table[logical]
            if self.pool.ref[old] > 1:
                b = self.pool.allocate()
                if b is None:
                    raise BlockError("no_blocks", "preemption required: no free blocks")
                self.pool.free(old)
                table[logical] = b
                new_block = b
                copy = (old, b)
        return table[logical] * B + offset, new_block, copy

    def free_request(self, rid: int) -> None:
        table = self._table(rid)
        del self.tables[rid]
        for b in table:
            self.pool.free(b)

    def share_prefix_blocks(self, src: int, dst: int, shared_len: int) -> None:
        """``dst`` gets the first ceil(shared_len / B) blocks of ``src``."""
        table = self._table(src)
        if shared_len < 0:
            raise BlockError("invalid", "shared_len must be >= 0")
        if dst in self.tables:
            raise BlockError("state", f"request {dst} already has a table")
        n = num_required_blocks(shared_len, self.block_size)
        if len(table) < n:
            raise BlockError("state", "source has fewer blocks than the shared length needs")
        for b in table[:n]:
            self.pool.add_ref(b)
        self.tables[dst] = list(table[:n])

    def fork(self, src: int, dst: int) -> None:
        """Beam-search fork (P3 §4): ``dst`` shares every block of ``src``."""
        table = self._table(src)
        self.share_prefix_blocks(src, dst, len(table) * self.block_size)

    def num_free(self) -> int:
        return len(self.pool.free_queue)

    def free_ids(self) -> list[int]:
        return list(self.pool.free_queue)

    def table(self, rid: int) -> list[int]:
        return list(self._table(rid))
