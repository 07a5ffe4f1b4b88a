"""CPU model of the decode split kernel's work partition, written from its
rules: the visible keys of all sequences (rows j0_b .. L_b - 1, j0_b =
max(0, L_b - 1 - W) with a window W, else 0; L_b = seqlens[b] clamped to
[0, T_cap], or with the appended token min(max(seqlens[b], 0), T_cap - 1) + 1)
are laid end to end, pre[b] = n_0 + ... + n_{b-1}; P = max(1, min(grid,
N / 64)) workgroups take the ranges [floor(w N / P), floor((w + 1) N / P));
a range's first segment starts at the sequence holding its first key (largest
b with pre[b] <= x), segments are walked in batches of 4 rows (rows past the
segment's end re-read its last row with zero weight), a segment's partial is
slot w - owner(pre[b]) of its sequence (owner(x) = floor(((x + 1) P - 1) / N),
the workgroup whose range holds flattened key x), and the range holding a
sequence's last key writes the segment count.

Checks, over random ragged batches, windows, appends and grid sizes: every
visible row is used exactly once and no row outside [j0_b, L_b) is read;
every range holds at least min(64, N) keys; segment slots are distinct and
below the per-sequence capacity ceil(T_cap / 64) + 1 that sizes the
workspace; each non-empty sequence gets its count and slots 0 .. count - 1."""
import random

import pytest

KMIN, U = 64, 4


def seg_cap(T_cap):
    return (T_cap + KMIN - 1) // KMIN + 1


def partition(lens, T_cap, win, app, grid):
    B = len(lens)
    L = [min(max(int(x), 0), T_cap - app) + app for x in lens]
    j0 = [0 if win < 0 else max(0, l - 1 - win) for l in L]
    pre = [0]
    for l, f in zip(L, j0):
        pre.append(pre[-1] + l - f)
    N = pre[B]
    P = max(1, min(grid, N // KMIN))
    used = {}
    slots = {}
    count = {}
    if N == 0:
        return L, j0, used, slots, count
    for w in range(P):
        lo, hi = w * N // P, (w + 1) * N // P
        assert hi - lo >= min(KMIN, N)

        def owner(x):
            return ((x + 1) * P - 1) // N

        def segment(x):
            a, b = 0, B - 1          # largest b with pre[b] <= x
            while a < b:
                mid = (a + b + 1) // 2
                if pre[mid] <= x:
                    a = mid
                else:
                    b = mid - 1
            return a, j0[a] + x - pre[a], j0[a] + min(hi, pre[a + 1]) - pre[a]

        b, j, jend = segment(lo)
        while True:
            for i in range(U):
                r = min(j + i, jend - 1)
                assert j0[b] <= r < L[b] <= T_cap, (b, r)
                if j + i < jend:
                    used[(b, j + i)] = used.get((b, j + i), 0) + 1
            if j + U < jend:
                j += U
                continue
            k = w - owner(pre[b])
            assert 0 <= k < seg_cap(T_cap)
            assert (b, k) not in slots
            slots[(b, k)] = w
            if pre[b] + jend - j0[b] == pre[b + 1]:
                count[b] = k + 1
            x = min(pre[b + 1], hi)
            if x >= hi:
                break
            b, j, jend = segment(x)
    return L, j0, used, slots, count


def check(lens, T_cap, win, app, grid):
    L, j0, used, slots, count = partition(lens, T_cap, win, app, grid)
    for b in range(len(lens)):
        for r in range(T_cap):
            want = 1 if j0[b] <= r < L[b] else 0
            assert used.get((b, r), 0) == want, (b, r)
        if L[b] > j0[b]:
            assert b in count
            assert all((b, k) in slots for k in range(count[b]))
            assert not any((b, k) in slots for k in range(count[b], seg_cap(T_cap)))
        else:
            assert b not in count


def test_d20_decode_shape():
    """The bench's d20 decode batch: 64 lengths in [1, 2048], 512 workgroups."""
    rng = random.Random(5)
    check([rng.randint(1, 2048) for _ in range(64)], 2048, -1, 0, 512)


@pytest.mark.parametrize("seed", range(40))
def test_random_batches(seed):
    rng = random.Random(seed)
    B = rng.randint(1, 90)
    T_cap = rng.choice([1, 2, 5, 40, 63, 64, 65, 130, 400, 2048])
    app = rng.randint(0, 1)
    win = rng.choice([-1, 0, 1, 3, 63, 64, 100])
    low = 0 if rng.random() < 0.5 else 1
    lens = [rng.randint(low, T_cap) for _ in range(B)]
    if rng.random() < 0.15:
        lens = [0] * B
    check(lens, T_cap, win, app, rng.choice([1, 3, 512, 1024]))


def test_workspace_slots_per_sequence_bound():
    """A sequence of T_cap visible keys split over ranges of exactly 64 keys
    that straddle its ends uses the most slots: ceil(T_cap / 64) + 1."""
    T_cap = 640
    lens = [32, T_cap, 32]     # offsets the long sequence by half a range
    L, j0, used, slots, count = partition(lens, T_cap, -1, 0, 1 << 20)
    assert count[1] == seg_cap(T_cap)
