"""CPU model of the dK/dV kernel's query-tile stream across work items,
written from the kernel's buffer rules: three LDS buffers hold query tiles,
the item whose first tile sits in buffer gb keeps tile qt0 + i in buffer
(gb + i) % 3, the next item's K rows and first two tiles are copied during the
current item's last tiles (K into its own staging region, tiles into the
buffers those tiles free), and its V rows go into the last tile's buffer once
that tile is done.  Checks that every tile a step reads has landed in the
buffer it reads, and that no copy targets a buffer still being read, for
random item sequences, ragged T, sliding windows (an item's query tiles
then end at the last tile that sees its keys) and grouped key/value heads
(an item's positions run over the G query heads that read its keys, position
n = g (qte - qt0) + t - qt0)."""
import random

import pytest

QT, KT, NB = 64, 128, 3


def run_stream(T, items, W=None, G=1):
    n_qt = (T + QT - 1) // QT
    qt0 = lambda it: items[it] * KT // QT  # noqa: E731

    def qte(it):
        if W is None:
            return n_qt
        return min(n_qt, (items[it] * KT + KT - 1 + W) // QT + 1)

    def npos(it):  # positions of an item
        return G * (qte(it) - qt0(it))

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
    issue(0, ("Q", cur, 0), set())
    if 1 < npos(cur):
        issue(1, ("Q", cur, 1), set())
    land()
    r = 0
    while True:
        N = npos(cur)
        ub2 = (gb + 2) % NB
        assert state["k"] == ("K", cur) and buf[ub2] == ("V", cur)
        assert buf[gb] == ("Q", cur, 0)
        if N > 1:
            assert buf[(gb + 1) % NB] == ("Q", cur, 1)
        if 2 < N:  # after the barrier that frees the V rows' buffer
            issue(ub2, ("Q", cur, 2), {gb, (gb + 1) % NB})
        nx, u = 0, gb
        for n in range(N):
            un = (u + 1) % NB
            if n > 0:
                land()
                u2, pos, busy = (un + 1) % NB, n + 2, {u, un}
                if pos < N:
                    issue(u2, ("Q", cur, pos), busy)
                elif nxt is not None and pos - N == nx and nx < 2 and nx < npos(nxt):
                    issue(u2, ("Q", nxt, nx), busy)
                    nx += 1
                if n == N - 1 and nxt is not None:
                    issue("k", ("K", nxt), busy)
            # a step reads position n (buffer u) and rows of position n + 1
            # (buffer un; across a query-head boundary too)
            assert buf[u] == ("Q", cur, n), (n, u, buf)
            if n + 1 < N:
                assert buf[un] == ("Q", cur, n + 1), (n, un, buf)
            u = un
        ulast = (gb + N - 1) % NB  # barrier: the last tile is done
        if nxt is None:
            break
        if N == 1:
            issue("k", ("K", nxt), set())
        issue(ulast, ("V", nxt), set())
        for j in range(nx, 2):
            if j < npos(nxt):
                issue((gb + N + j) % NB, ("Q", nxt, j), set())
        land()
        gb, cur, r = (gb + N) % NB, nxt, r + 1
        nxt = r + 1 if r + 1 < len(items) else None


@pytest.mark.parametrize("T", [1, 5, 63, 64, 65, 100, 127, 128, 129, 192, 200, 256, 257, 300,
                               384, 512, 1000, 2048])
@pytest.mark.parametrize("W", [None, 0, 1, 5, 63, 64, 100, 127, 128, 200, 1000])
def test_stream_buffers(T, W):
    rng = random.Random(T * 131 + (W if W is not None else -1))
    n_kt = (T + KT - 1) // KT
    for _ in range(40):
        items = [rng.randrange(n_kt) for _ in range(rng.randint(1, 12))]
        run_stream(T, items, W, G=rng.choice([1, 1, 2, 3, 5]))


@pytest.mark.parametrize("nt", [1, 2, 3, 5, 32])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 8])
def test_position_two_ahead_without_division(nt, G):
    """The kernel finds the (query head, tile) of position n + 2 from that of
    position n by at most two wrap-arounds of t; this equals divmod."""
    qt0 = 7
    qte = qt0 + nt
    for n in range(G * nt):
        g, t = divmod(n, nt)
        t += qt0
        if n + 2 >= G * nt:
            continue
        g2, t2 = g, t + 2
        if t2 >= qte:
            t2, g2 = t2 - nt, g2 + 1
        if t2 >= qte:
            t2, g2 = t2 - nt, g2 + 1
        assert (g2, t2 - qt0) == divmod(n + 2, nt)
