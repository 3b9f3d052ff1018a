"""Host logic of the decode GEMM's stream-K schedule (no GPU work): the
iteration ranges of the workgroups are contiguous, cover every (tile, k-step)
iteration exactly once, leave empty ranges only at the end, report as many
partial slots as the most-cut tile needs, and are balanced by time (k-steps
plus a fixed cost per tile touched) rather than by count."""
import ctypes

import pytest

I64, I32 = ctypes.c_int64, ctypes.c_int32


class SkSched(ctypes.Structure):
    _fields_ = [("T", I64), ("G", I64), ("nk", I64), ("ntn", I64), ("bm", I64), ("bn", I64),
                ("slots", I64), ("wide", I32), ("dp", I32), ("tiles", I64), ("mt", I64),
                ("band", I64), ("bnd", I32 * 257), ("slot0", ctypes.c_int16 * 256)]


@pytest.fixture(scope="module")
def sched():
    from throughput_oriented_offloaded_amd import _lib as L
    f = getattr(L._L, "_ZN2fg4gemm11sk_scheduleElll")
    f.restype, f.argtypes = SkSched, [I64, I64, I64]
    return f


SHAPES = [(144, 36864, 12288), (144, 12288, 12288), (144, 49152, 12288), (144, 12288, 49152),
          (144, 50272, 12288), (128, 6144, 2048), (256, 27648, 9216), (4, 2304, 768), (33, 768, 3072),
          (144, 21504, 7168), (96, 1024, 64), (1, 64, 64)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_ranges_cover_every_iteration_once(sched, M, N, K):
    sc = sched(M, N, K)
    assert not sc.dp
    G, T, nk = sc.G, sc.T, sc.nk
    b = list(sc.bnd)[:G + 1]
    assert b[0] == 0 and b[-1] == T
    assert all(b[i] <= b[i + 1] for i in range(G))
    lens = [b[i + 1] - b[i] for i in range(G)]
    first_empty = next((i for i, l in enumerate(lens) if l == 0), G)
    assert all(l == 0 for l in lens[first_empty:])          # empty ranges only at the end
    # segments per tile: the owners of its iterations are consecutive workgroups
    owner = {}
    for g in range(G):
        for x in range(b[g], b[g + 1]):
            owner.setdefault(x // nk, set()).add(g)
    assert len(owner) == sc.tiles
    most = 1
    for t, gs in owner.items():
        assert sorted(gs) == list(range(min(gs), max(gs) + 1))
        most = max(most, len(gs))
    assert sc.slots == most
    # the slot of each workgroup's first segment is its rank among the
    # workgroups of that tile; a segment starting at a tile's first k-step is
    # the tile's first (slot 0)
    for g in range(first_empty):
        t = b[g] // nk
        rank = sorted(owner[t]).index(g)
        assert sc.slot0[g] == (0 if b[g] % nk == 0 else rank)
        if b[g] % nk == 0:
            assert rank == 0


@pytest.mark.parametrize("M,N,K", [(144, 36864, 12288), (144, 12288, 12288), (144, 49152, 12288),
                                   (144, 12288, 49152)])
def test_ranges_balanced_by_time(sched, M, N, K):
    """At the OPT-175B shapes (R = 12 k-steps per tile touched), no
    workgroup's estimated time exceeds the uniform split's, and the spread
    between the busiest and the idlest is within one segment cost."""
    sc = sched(M, N, K)
    G, T, nk, R = sc.G, sc.T, sc.nk, 12
    b = list(sc.bnd)[:G + 1]

    def cost(lo, hi):
        return 0 if hi <= lo else (hi - lo) + R * ((hi - 1) // nk - lo // nk + 1)
    bal = [cost(b[g], b[g + 1]) for g in range(G)]
    uni = [cost(g * T // G, (g + 1) * T // G) for g in range(G)]
    assert max(bal) <= max(uni)
    assert max(bal) - min(c for c in bal if c) <= R + 1
