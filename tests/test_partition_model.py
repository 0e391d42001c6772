"""The weighted stream-K cut of the split pass and of extend, modelled on the
host: key ranges laid end to end, each weighing its tiles plus a fixed piece
cost in front of its first tile, cut into W equal ranges of units and walked
the way the kernels walk them (decode_split_kernel / extend_kernel).  Checks
the properties the merge relies on: every tile is computed exactly once, the
owner of a range's first tile records the ranges covering it, every range
between those owners either holds a piece of it in the slot the merge reads
or is empty, and no range writes two pieces to one slot."""
import random

import pytest


def walk(tiles, hm, W, A):
    """tiles[b]: tiles per segment of sequence b; hm segments per sequence
    (kv heads of one stream).  Returns the pieces per segment, the records
    and the empty ranges."""
    units = [(t + A) * hm if t > 0 else 0 for t in tiles]
    pfx = [0]
    for u in units:
        pfx.append(pfx[-1] + u)
    N = pfx[-1]

    def start(w):
        return w * N // W

    def owner(t):                      # the largest w with start(w) <= t
        return ((t + 1) * W + N - 1) // N - 1

    pieces, recs, empty, slots = {}, {}, set(), {}
    for w in range(W):
        r0, r1 = start(w), start(w + 1)
        if r0 >= r1:
            empty.add(w)
            continue
        b = next(i for i in range(len(tiles)) if units[i] and pfx[i] <= r0 < pfx[i + 1])
        seq_start, pos, slot = pfx[b], r0, 0
        while pos < r1:
            n = tiles[b]
            nu = n + A
            h = (pos - seq_start) // nu
            seg_end = seq_start + (h + 1) * nu
            u0 = seg_end - n                       # unit of the first tile
            i0 = max(pos - u0, 0)
            cnt = min(r1, seg_end) - u0 - i0
            if cnt <= 0:                           # the range ends in the piece cost
                break
            assert 0 <= i0 < n and 1 <= cnt <= n - i0
            complete = i0 == 0 and cnt == n
            if i0 == 0:
                recs[(b, h)] = (w, w if complete else owner(seg_end - 1), slot)
            pieces.setdefault((b, h), []).append((w, slot, i0, cnt, complete))
            if not complete:
                assert (w, slot) not in slots
                slots[(w, slot)] = (b, h)
            pos, slot = min(r1, seg_end), 1
            if pos < r1 and pos == seq_start + nu * hm:
                seq_start = pos
                b += 1
                while tiles[b] == 0:
                    b += 1
    return pieces, recs, empty, slots


def check(tiles, hm, W, A):
    pieces, recs, empty, slots = walk(tiles, hm, W, A)
    for b, t in enumerate(tiles):
        for h in range(hm):
            if t == 0:
                assert (b, h) not in pieces
                continue
            ps = pieces[(b, h)]
            spans = sorted((i0, i0 + cnt) for _, _, i0, cnt, _ in ps)
            assert spans[0][0] == 0 and spans[-1][1] == t
            assert all(a[1] == c[0] for a, c in zip(spans, spans[1:]))
            w0, w1, slot0 = recs[(b, h)]
            if len(ps) == 1 and ps[0][4]:
                assert w0 == w1 == ps[0][0]
                continue
            seen = []
            for k, w in enumerate(range(w0, w1 + 1)):
                if w in empty:
                    continue                       # its slot 0 holds lse = -inf
                assert slots.get((w, slot0 if k == 0 else 0)) == (b, h)
                seen.append(w)
            assert sorted(seen) == sorted(p[0] for p in ps)


@pytest.mark.parametrize("A", [0, 1, 3, 4, 6])
def test_weighted_cut_covers_every_tile_once(A):
    rng = random.Random(1000 + A)
    for _ in range(400):
        tiles = [rng.choice([0, 0, 1, 2, 3, rng.randint(1, 40), rng.randint(1, 300)])
                 for _ in range(rng.randint(1, 40))]
        if not any(tiles):
            continue
        check(tiles, rng.choice([1, 1, 2, 4, 8]),
              rng.choice([1, 2, 3, 7, 8, 16, 31, 64, 224, 1000]), A)


def test_weighted_cut_shifts_tiles_away_from_short_segments():
    """With a piece cost, a range full of short segments holds fewer tiles
    than one inside a long segment."""
    tiles = [1] * 64 + [640]
    W = 8
    pieces, _, _, _ = walk(tiles, 1, W, 4)
    per_range = [0] * W
    for ps in pieces.values():
        for w, _, _, cnt, _ in ps:
            per_range[w] += cnt
    assert per_range[0] < per_range[-1]
    plain, _, _, _ = walk(tiles, 1, W, 0)
    per_plain = [0] * W
    for ps in plain.values():
        for w, _, _, cnt, _ in ps:
            per_plain[w] += cnt
    assert per_range[0] < per_plain[0]
