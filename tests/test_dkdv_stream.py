"""CPU model of the dK/dV kernel's query-tile stream across work items,
written from the kernel's buffer rules: three LDS buffers hold query tiles,
the item whose first tile sits in buffer gb keeps tile qt0 + i in buffer
(gb + i) % 3, the next item's K rows and first two tiles are copied during the
current item's last tiles (K into its own staging region, tiles into the
buffers those tiles free), and its V rows go into the last tile's buffer once
that tile is done.  Checks that every tile a step reads has landed in the
buffer it reads, and that no copy targets a buffer still being read, for
random item sequences, ragged T and sliding windows (an item's query tiles
then end at the last tile that sees its keys)."""
import random

import pytest

QT, KT, NB = 64, 128, 3


def run_stream(T, items, W=None):
    n_qt = (T + QT - 1) // QT
    qt0 = lambda it: items[it] * KT // QT  # noqa: E731

    def qte(it):
        if W is None:
            return n_qt
        return min(n_qt, (items[it] * KT + KT - 1 + W) // QT + 1)

    buf = [None] * NB
    state = {"k": None}
    pending = []

    def land():  # wait for every copy issued so far, then a barrier
        for reg, tag in pending:
            if reg == "k":
                state["k"] = tag
            else:
                buf[reg] = tag
        pending.clear()

    def issue(reg, tag, busy):
        assert reg not in busy, (reg, tag, busy)
        pending.append((reg, tag))

    cur, gb = 0, 0
    nxt = 1 if len(items) > 1 else None
    issue("k", ("K", cur), set())
    issue(2, ("V", cur), set())
    issue(0, ("Q", cur, qt0(cur)), set())
    if qt0(cur) + 1 < qte(cur):
        issue(1, ("Q", cur, qt0(cur) + 1), set())
    land()
    r = 0
    while True:
        q0, E = qt0(cur), qte(cur)
        nt = E - q0
        ub2 = (gb + 2) % NB
        assert state["k"] == ("K", cur) and buf[ub2] == ("V", cur)
        assert buf[gb] == ("Q", cur, q0)
        if nt > 1:
            assert buf[(gb + 1) % NB] == ("Q", cur, q0 + 1)
        if q0 + 2 < E:  # after the barrier that frees the V rows' buffer
            issue(ub2, ("Q", cur, q0 + 2), {gb, (gb + 1) % NB})
        nx, u = 0, gb
        for t in range(q0, E):
            un = (u + 1) % NB
            if t > q0:
                land()
                u2, pos, busy = (un + 1) % NB, t + 2, {u, un}
                if pos < E:
                    issue(u2, ("Q", cur, pos), busy)
                elif nxt is not None and pos - E == nx and nx < 2 and qt0(nxt) + nx < qte(nxt):
                    issue(u2, ("Q", nxt, qt0(nxt) + nx), busy)
                    nx += 1
                if t == E - 1 and nxt is not None:
                    issue("k", ("K", nxt), busy)
            # a step reads tile t (buffer u) and rows of tile t + 1 (buffer un)
            assert buf[u] == ("Q", cur, t), (t, u, buf)
            if t + 1 < E:
                assert buf[un] == ("Q", cur, t + 1), (t, un, buf)
            u = un
        ulast = (gb + nt - 1) % NB  # barrier: the last tile is done
        if nxt is None:
            break
        if nt == 1:
            issue("k", ("K", nxt), set())
        issue(ulast, ("V", nxt), set())
        for j in range(nx, 2):
            if qt0(nxt) + j < qte(nxt):
                issue((gb + nt + j) % NB, ("Q", nxt, qt0(nxt) + j), set())
        land()
        gb, cur, r = (gb + nt) % NB, nxt, r + 1
        nxt = r + 1 if r + 1 < len(items) else None


@pytest.mark.parametrize("T", [1, 5, 63, 64, 65, 100, 127, 128, 129, 192, 200, 256, 257, 300,
                               384, 512, 1000, 2048])
@pytest.mark.parametrize("W", [None, 0, 1, 5, 63, 64, 100, 127, 128, 200, 1000])
def test_stream_buffers(T, W):
    rng = random.Random(T * 131 + (W if W is not None else -1))
    n_kt = (T + KT - 1) // KT
    for _ in range(40):
        items = [rng.randrange(n_kt) for _ in range(rng.randint(1, 12))]
        run_stream(T, items, W)
