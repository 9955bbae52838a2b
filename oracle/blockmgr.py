"""Reference model of the block manager's bookkeeping (plain Python).

Test infrastructure only (see the package docstring).  It restates, in the
simplest data structures, the per-request and per-block state and the growth
protocol of [Slides] "PagedAttention：让 KV cache 按需生长":

  * state ("引用计数管理“谁还在读”，长度管理“哪里能写”"): per request a block
    table and a length; per block a refcount (tables holding it, not tokens);
    a FIFO free queue of blocks whose refcount is 0;
  * growth ("先确保分配成功，再改变可见状态"): if the tail is full, take a
    fresh block and append it; else if the tail is shared (refcount > 1), take
    a fresh block, copy the tail's valid slots into it, drop one reference
    from the old tail and point the table at the copy; then write;
  * capacity is checked before anything changes ("三个空闲块，四个请求同时
    跨边界"): a call that cannot get all its blocks changes nothing;
  * release ("请求结束，块就能交给下一位"): drop the table; blocks whose
    refcount reaches 0 go back to the free queue (no prefix cache);
  * rollback ([Serving] §5: speculative decoding writes KV positions that
    may be taken back): shorten a request; table entries past the new block
    count drop one reference each, exactly as in release.

Readings: requests in one decode step are served in the order given, so when
several share a partly filled tail, the earlier ones copy and the last one
left writes in place.  Request ids count up from 0.  Blocks released by a
release or a rollback join the free queue in table order.  A rollback keeps
the (now partly valid) tail block as it is: the slots past the new length
are dead and the next growth writes over them, or copies only the valid
slots first if the tail is shared.
"""

from collections import deque


class NoSpace(Exception):
    """The pool cannot supply the blocks a call needs; nothing changed."""


class BlockManagerModel:
    def __init__(self, num_blocks, block_size, max_blocks_per_seq, free_order=None):
        self.B = block_size
        self.MB = max_blocks_per_seq
        self.refcount = [0] * num_blocks
        self.free = deque(range(num_blocks) if free_order is None else [int(b) for b in free_order])
        self.tables = {}
        self.lengths = {}
        self.next_id = 0

    # -- queries
    def num_free(self):
        return len(self.free)

    def blocks_of(self, req):
        return list(self.tables[req])

    # -- lifecycle
    def add_request(self):
        rid = self.next_id
        self.next_id += 1
        self.tables[rid] = []
        self.lengths[rid] = 0
        return rid

    def fork(self, parent):
        rid = self.next_id
        self.next_id += 1
        self.tables[rid] = list(self.tables[parent])
        self.lengths[rid] = self.lengths[parent]
        for b in self.tables[rid]:
            self.refcount[b] += 1
        return rid

    def release(self, req):
        for b in self.tables.pop(req):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)
        del self.lengths[req]

    def truncate(self, req, new_length):
        """Roll request `req` back to its first new_length tokens."""
        if not 0 <= new_length <= self.lengths[req]:
            raise ValueError("new length outside [0, length]")
        keep = -(-new_length // self.B)
        table = self.tables[req]
        for b in table[keep:]:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)
        del table[keep:]
        self.lengths[req] = new_length

    # -- growth
    def _blocks_needed(self, length, extra, tail_refcount):
        """Fresh blocks to grow a request of `length` tokens by `extra`."""
        partial_tail = length % self.B != 0
        copy = partial_tail and tail_refcount > 1
        now = -(-length // self.B)
        after = -(-(length + extra) // self.B)
        return (1 if copy else 0) + (after - now), copy

    def _take(self):
        b = self.free.popleft()
        self.refcount[b] = 1
        return b

    def _grow(self, req, extra):
        """Apply growth (blocks known to be available); returns the copy or None."""
        table, length = self.tables[req], self.lengths[req]
        copy = None
        if extra == 0:
            return None
        if length % self.B != 0 and self.refcount[table[-1]] > 1:
            old = table[-1]
            new = self._take()
            self.refcount[old] -= 1
            table[-1] = new
            copy = (old, new, length % self.B)
        while len(table) < -(-(length + extra) // self.B):
            table.append(self._take())
        self.lengths[req] = length + extra
        return copy

    def reserve(self, req, extra):
        length = self.lengths[req]
        if -(-(length + extra) // self.B) > self.MB:
            raise ValueError("request would exceed its table width")
        tail_rc = self.refcount[self.tables[req][-1]] if self.tables[req] else 0
        need, _ = self._blocks_needed(length, extra, tail_rc)
        if extra > 0 and need > len(self.free):
            raise NoSpace(f"need {need}, have {len(self.free)}")
        return self._grow(req, extra)

    def prepare_append(self, reqs):
        """One token per request, in order: (positions, [copies])."""
        return self.prepare_extend(reqs, 1)

    def prepare_extend(self, reqs, extra):
        """`extra` tokens per request, in order: (start positions, [copies]).

        All or nothing, like a single token: the blocks of the whole step are
        counted before any request grows.
        """
        if extra < 1:
            raise ValueError("extra must be >= 1")
        if len(set(reqs)) != len(reqs):
            raise ValueError("a request is listed twice")
        # dry run: who copies, and how many fresh blocks in all
        rc = {}
        need = 0
        for r in reqs:
            length = self.lengths[r]
            if -(-(length + extra) // self.B) > self.MB:
                raise ValueError("request would exceed its table width")
            tail = self.tables[r][-1] if self.tables[r] else None
            cur = rc.get(tail, self.refcount[tail]) if tail is not None else 0
            k, copy = self._blocks_needed(length, extra, cur)
            need += k
            if copy:
                rc[tail] = cur - 1
        if need > len(self.free):
            raise NoSpace(f"need {need}, have {len(self.free)}")
        positions, copies = [], []
        for r in reqs:
            positions.append(self.lengths[r])
            c = self._grow(r, extra)
            if c is not None:
                copies.append(c)
        return positions, copies
