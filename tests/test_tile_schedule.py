"""CPU model of the tile kernel's weight-ring schedule (hc_kernels.hip,
hc_tile_kernel): per wave, RING slots of LDS hold W units; the prologue loads
units 0..RING-1 of the first tile, each unit is read once and its slot is
refilled with the unit RING positions later (continuing into the next tile).
For every shape the kernel instantiates and several tiles per workgroup, the
model checks that each read finds the unit it wants and that, at the
vector-memory wait before it, at least LOADS * (RING - 1) loads were issued
after that unit's loads (the wait leaves only that many in flight, and loads
complete in issue order)."""
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
    return U, LOADS, SLOT, RING


def simulate(N, V, CS, tiles):
    U, LOADS, SLOT, RING = ring_shape(N, V, CS)
    assert 1 <= RING and RING * SLOT <= TILE_RING_BYTES
    slots = [None] * RING
    ops = []

    def issue(tile, u, slot):
        ops.extend([(tile, u)] * LOADS)
        slots[slot] = (tile, u)

    for u in range(RING):
        issue(0, u, u)
    ring_pos = 0
    for k in range(tiles):
        for u in range(U):
            slot = ring_pos + u % RING
            slot = slot - RING if slot >= RING else slot
            last = max(i for i, o in enumerate(ops) if o == (k, u))
            assert len(ops) - 1 - last >= LOADS * (RING - 1), (k, u)
            assert slots[slot] == (k, u), (k, u, slots[slot])
            nu = u + RING
            if nu < U:
                issue(k, nu, slot)
            else:
                issue(k + 1, nu - U, slot)
        ring_pos = (ring_pos + U) % RING


@pytest.mark.parametrize("N,V", list(itertools.product([1, 2, 4], [4, 8])))
def test_ring_schedule(N, V):
    for CS in range(1, 9):
        for tiles in (1, 2, 3, 5):
            simulate(N, V, CS, tiles)


def test_ring_fits_lds():
    # eight waves' rings plus the kernel's small reduction arrays stay within 160 KiB
    for N, V, CS in itertools.product([1, 2, 4], [4, 8], range(1, 9)):
        U, LOADS, SLOT, RING = ring_shape(N, V, CS)
        assert 8 * RING * SLOT <= 144 * 1024
