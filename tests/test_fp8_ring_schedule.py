"""CPU model of the FP8 attention kernel's K/V ring: which tile copies each
wavefront has issued and awaited when a tile is read.

The kernel (attn_fp8_kernel) keeps an eight-tile ring.  Leading wavefronts
issue the copies of tile t + 6 at the start of half step 2t, read K of tile
t + 1 in half step 2t and V^T of tile t in half step 2t + 1; trailing
wavefronts run the same blocks half a step later (copies of tile t + 7 in
half step 2t + 2).  Only odd half steps end with a wait (at most 8 copies of
this wavefront outstanding), every half step with a barrier.  Copies
complete in issue order.  The model checks, for every tile count, that each
tile read has landed for every wavefront, and that no copy overwrites a
buffer before its last read -- with copies issued for every tile, as the
kernel does, and (as a regression of a tail race) that skipping the copies
past the last tile breaks the first property."""
import pytest

BUF, AHEAD, WAIT = 8, 6, 8      # ring tiles, copy distance of the leading role, vmcnt of the odd ends
COPIES = 2                      # copies per tile and wavefront (K and V^T)


def schedule(nt, trailing, issue_past_end):
    """Events of one wavefront: ('copy', tile, half_step), ('read', tile,
    half_step), ('wait', None, half_step) in program order."""
    ev = []
    issue = lambda t, h: ev.append(("copy", t, h)) if (issue_past_end or t < nt) else None
    for t in range(BUF - 2):
        issue(t, -1)
    ev.append(("wait0", None, -1))
    if not trailing:
        for t in range(nt):
            issue(t + AHEAD, 2 * t)
            ev.append(("read", t + 1, 2 * t))          # K of the next tile (past the end: masked)
            ev.append(("read", t, 2 * t + 1))          # V^T of this tile
            ev.append(("wait", None, 2 * t + 1))
    else:
        issue(AHEAD, 0)
        for t in range(nt):
            ev.append(("read", t + 1, 2 * t + 1))
            ev.append(("wait", None, 2 * t + 1))
            issue(t + AHEAD + 1, 2 * t + 2)
            ev.append(("read", t, 2 * t + 2))
    return ev


def landed_before(ev):
    """half step h -> set of tiles whose copies (this wavefront's) have all
    completed at the last wait before half step h begins."""
    issued, done, out, last = [], 0, {}, set()
    for kind, t, h in ev:
        if kind == "copy":
            issued.append(t)
        elif kind in ("wait", "wait0"):
            # completed copies never un-complete: at least the earlier count
            done = max(done, len(issued) * COPIES - (0 if kind == "wait0" else WAIT))
            n_tiles = max(done, 0) // COPIES
            last = set(issued[:n_tiles])
            out[h + 1] = last
    return out


def check(nt, issue_past_end):
    bad = []
    for trailing in (False, True):
        ev = schedule(nt, trailing, issue_past_end)
        landed = landed_before(ev)
        for kind, t, h in ev:
            if kind == "read" and t < nt:
                # the latest wait that ends at or before half step h - 1
                ready = max((k for k in landed if k <= h), default=None)
                if ready is None or t not in landed[ready]:
                    bad.append((trailing, t, h))
    return bad


def overwrite_violations(nt):
    """A copy of tile u goes into the buffer of tile u - BUF; that tile's last
    read (either role) must come in an earlier half step."""
    last_read = {}
    for trailing in (False, True):
        for kind, t, h in schedule(nt, trailing, True):
            if kind == "read":
                last_read[t] = max(last_read.get(t, -9), h)
    out = []
    for trailing in (False, True):
        for kind, t, h in schedule(nt, trailing, True):
            if kind == "copy" and t >= BUF and last_read.get(t - BUF, -9) >= h:
                out.append((trailing, t, h))
    return out


@pytest.mark.parametrize("nt", list(range(1, 40)))
def test_every_read_tile_has_landed(nt):
    assert check(nt, issue_past_end=True) == []
    assert overwrite_violations(nt) == []


def test_skipping_copies_past_the_end_races():
    """The schedule before the fix: from 7 tiles on, the last tiles are read
    before the wait covers them."""
    assert all(check(nt, issue_past_end=False) == [] for nt in range(1, 7))
    assert all(check(nt, issue_past_end=False) != [] for nt in range(7, 40))
