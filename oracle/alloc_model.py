"""Model of the exact transactional fixed-block allocator (oracle; test
infrastructure only).

lucebox#555, Summary, names the allocator's properties: exact fixed-size
blocks, transactional allocation, stale-handle detection, immediate release.
TensorFold#1156, Design / Host, takes K/V pages from the bottom of its arena.
This model makes each property concrete, with these readings:

* exact: ``n_free + n_used == n_blocks`` at all times; a request for more
  blocks than are free fails and changes nothing;
* transactional: a call allocates all ``n`` blocks or none, and frees all the
  given handles or none;
* lowest free index first (pages from the bottom), so the index sequence of
  any alloc/free history is unique;
* a handle is ``(generation << 32) | index``; every block starts at
  generation 1; a successful free bumps the block's generation (2**32 - 1
  wraps to 1), so every earlier handle of that block is stale from then on;
* free rejects, before releasing anything: an index out of range, a
  generation that is not the block's current one, a block that is not
  allocated, and the same block twice in one call.
"""

OK = "ok"
NOMEM = "nomem"
STALE = "stale"
INVALID = "invalid"

GEN_START = 1
GEN_MOD = 1 << 32


def handle(gen: int, index: int) -> int:
    return (gen << 32) | index


def split(h: int):
    return h >> 32, h & 0xFFFFFFFF


class AllocModel:
    def __init__(self, n_blocks: int):
        if n_blocks <= 0:
            raise ValueError("n_blocks must be positive")
        self.n_blocks = n_blocks
        self.free = set(range(n_blocks))
        self.gen = [GEN_START] * n_blocks

    @property
    def n_free(self) -> int:
        return len(self.free)

    @property
    def n_used(self) -> int:
        return self.n_blocks - len(self.free)

    def alloc(self, n: int):
        """Returns (status, handles, indices)."""
        if n < 0:
            return INVALID, [], []
        if n > len(self.free):
            return NOMEM, [], []
        idx = sorted(self.free)[:n]
        for i in idx:
            self.free.discard(i)
        return OK, [handle(self.gen[i], i) for i in idx], idx

    def free_handles(self, handles):
        """Returns status; on any failure nothing is freed."""
        seen = set()
        for h in handles:
            if h < 0 or h >= (1 << 64):
                return INVALID
            g, i = split(h)
            if i >= self.n_blocks:
                return INVALID
            if g != self.gen[i] or i in self.free or i in seen:
                return STALE
            seen.add(i)
        for i in seen:
            self.free.add(i)
            g = (self.gen[i] + 1) % GEN_MOD
            self.gen[i] = g if g != 0 else GEN_START
        return OK
