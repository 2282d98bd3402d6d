"""CPU model of the tile kernel's per-wave load schedule (hc_kernels.hip,
hc_tile_kernel), checked for every shape the kernel instantiates and several
tiles per workgroup.

Per wave, the LDS ring area holds RING slots of LOADS 1 KiB blocks. In a tile's
projection unit u reads slot u % RING and, while u + RING < U, refills that slot
with unit u + RING of the same tile. After the projection the drained area takes
the next tile's rows of the first STAGED column steps (one 1 KiB block per
stream and step, by direct loads); pass 2 reads step j < STAGED back from it
and, after the last staged step, reloads the ring with the next tile's units
0 .. RING - 1; the other steps load their rows from HBM into registers.

A wait "at most w outstanding" completes every load except the last w issued
(loads complete in issue order; stores only add to the count, so they are left
out, which is the conservative side). The model applies a direct load's LDS
write when it completes and checks, at every read, that the block holds what
the kernel expects and that no load still in flight targets it."""
import itertools

import pytest

TILE_RING_BYTES = 18 * 1024   # per wave, as in the kernel


def ring_shape(N, V, CS):
    M = 2 * N + N * N
    G = (M + 3) // 4
    STEP = 16 * V
    U = CS * N
    UNIT = 4 * G * STEP * 2
    LOADS = (UNIT + 1023) // 1024
    SLOT = LOADS * 1024
    RING = min(min(TILE_RING_BYTES // SLOT, 8), U)
    STAGED = min(RING * SLOT // (N * 1024), CS)
    return U, LOADS, SLOT, RING, STAGED


def tile_unit_wait(u, U, RING, LOADS):
    """The kernel's wait before unit u (same formula as tile_unit_wait there)."""
    after = LOADS * (RING - 1 - u) + LOADS * min(u, U - RING) if u < RING \
        else LOADS * min(RING - 1, U - 1 - u)
    return min(after, 63)


class Wave:
    def __init__(self, blocks):
        self.ops = []        # issued loads: (tag, lds block or None)
        self.done = 0        # loads [0, done) have completed
        self.lds = [None] * blocks

    def issue(self, tag, block=None):
        self.ops.append((tag, block))

    def wait(self, at_most):
        target = max(len(self.ops) - at_most, self.done)
        for tag, block in self.ops[self.done:target]:
            if block is not None:
                self.lds[block] = tag
        self.done = target

    def complete(self, tag):
        return all(i < self.done for i, (t, _) in enumerate(self.ops) if t == tag)

    def read(self, block, want):
        assert self.lds[block] == want, (block, self.lds[block], want)
        pending = [t for t, b in self.ops[self.done:] if b == block]
        assert not pending, (block, pending)


def simulate(N, V, CS, tiles):
    U, LOADS, SLOT, RING, STAGED = ring_shape(N, V, CS)
    assert 1 <= RING and RING * SLOT <= TILE_RING_BYTES
    assert 1 <= STAGED <= CS and STAGED * N * 1024 <= RING * SLOT
    w = Wave(RING * LOADS)

    def issue_unit(k, u):
        for q in range(LOADS):
            w.issue(("W", k, u, q), (u % RING) * LOADS + q)

    for u in range(RING):                     # prologue of the first tile
        issue_unit(0, u)
    for j, i in itertools.product(range(CS), range(N)):
        w.issue(("row", 0, j, i))
    for k in range(tiles):
        for u in range(U):                    # projection
            w.wait(tile_unit_wait(u, U, RING, LOADS))
            for q in range(LOADS):
                assert w.complete(("W", k, u, q)), (k, u, q)
                w.read((u % RING) * LOADS + q, ("W", k, u, q))
            if u + RING < U:
                issue_unit(k, u + RING)
        for j in range(CS):                   # layer_out (fused mode)
            w.issue(("lo", k, j))
        for j, i in itertools.product(range(STAGED), range(N)):
            w.issue(("row", k + 1, j, i), j * N + i)
        for j in range(CS):                   # pass 2
            if j < STAGED:
                w.wait((STAGED - 1 - j) * N)
                for i in range(N):
                    assert w.complete(("row", k + 1, j, i))
                    w.read(j * N + i, ("row", k + 1, j, i))
                if j == STAGED - 1:
                    for u in range(RING):
                        issue_unit(k + 1, u)
            else:
                for i in range(N):
                    w.issue(("row", k + 1, j, i))
    w.wait(0)
    assert w.done == len(w.ops)


@pytest.mark.parametrize("N,V", list(itertools.product([1, 2, 4], [4, 8])))
def test_tile_schedule(N, V):
    for CS in range(1, 9):
        for tiles in (1, 2, 3, 5):
            simulate(N, V, CS, tiles)


def test_model_catches_a_short_wait():
    # the uniform wait of a ring that refills into the next tile is too loose
    # for this schedule's last units: the model must reject it
    U, LOADS, SLOT, RING, STAGED = ring_shape(4, 4, 8)
    w = Wave(RING * LOADS)
    for u in range(RING):
        for q in range(LOADS):
            w.issue(("W", 0, u, q), (u % RING) * LOADS + q)
    with pytest.raises(AssertionError):
        for u in range(U):
            w.wait(LOADS * (RING - 1))
            for q in range(LOADS):
                assert w.complete(("W", 0, u, q))
                w.read((u % RING) * LOADS + q, ("W", 0, u, q))
            if u + RING < U:
                for q in range(LOADS):
                    w.issue(("W", 0, u + RING, q), (u % RING) * LOADS + q)


def test_ring_fits_lds():
    # eight waves' rings plus the kernel's small reduction arrays stay within 160 KiB
    for N, V, CS in itertools.product([1, 2, 4], [4, 8], range(1, 9)):
        U, LOADS, SLOT, RING, STAGED = ring_shape(N, V, CS)
        assert 8 * RING * SLOT <= 144 * 1024
