"""Pins of the oracle's verify page bookkeeping (``ora_book_step``) on the CPU.

The bookkeeping follows "r9700-stack v0.2.4: one GDN state page per
request": section "What it does" (two record slots, a flag word holding the
live slot, a parity and a done counter; replay of the accepted rows of the
previous step) and section "A defect found and fixed before the tag" (the
conv buffer rolls by the rows the record holds).  It is pinned here against
values derived by hand and against the committed-stream semantics of verify
(every committed row is the previous step's candidate 0..a, so the window a
step reads is the last W-1 rows of the committed stream), computed by brute
force from a plain list of rows.
"""
import numpy as np
import pytest

W, N_SPEC = 4, 7
ROWS = W - 1 + N_SPEC


def buf(rows=ROWS, C=2, base=0.0):
    """A conv buffer whose entries name their row: row r channel c = base + 10 r + c."""
    return base + 10.0 * np.arange(rows)[:, None] + np.arange(C)[None, :]


def cand(n, step, C=2):
    """Candidate rows of a step, distinct from every buffer value: -(1000 step + 10 i + c) - 1."""
    return -(1000.0 * step + 10.0 * np.arange(n)[:, None] + np.arange(C)[None, :]) - 1.0


def test_hand_derived_steps(ora):
    hdr = np.zeros(4, np.uint32)
    cb = buf()
    # step 1 on a fresh page: parity 1, nothing to replay, acceptance ignored
    e, hdr, cb, info = ora.book_step(W, N_SPEC, hdr, cb, cand(8, 1), num_accepted=5, parity=1)
    assert e == 0 and info == (0, 0, 0, 1)
    assert list(hdr) == [1 | 2, 0, 8, 0]
    np.testing.assert_array_equal(cb[:2], buf()[1:3])           # old rows 1, 2
    np.testing.assert_array_equal(cb[2:10], cand(8, 1))
    # step 2: parity 0, 3 drafts accepted -> replay slot 1 rows 0..3, write slot 0
    e, hdr, cb, info = ora.book_step(W, N_SPEC, hdr, cb, cand(8, 2), num_accepted=3, parity=0)
    assert e == 0 and info == (3, 4, 1, 0)
    assert list(hdr) == [0 | 0, 8, 8, 3]
    # window of step 2 was rows 3..5 = [cand1[1], cand1[2], cand1[3]]; kept rows 4, 5
    np.testing.assert_array_equal(cb[:2], cand(8, 1)[2:4])
    np.testing.assert_array_equal(cb[2:10], cand(8, 2))
    # step 3: three candidates, 7 drafts accepted (all of step 2's)
    e, hdr, cb, info = ora.book_step(W, N_SPEC, hdr, cb, cand(3, 3), num_accepted=7, parity=1)
    assert e == 0 and info == (7, 8, 0, 1)
    assert list(hdr) == [1 | 2, 8, 3, 7]
    np.testing.assert_array_equal(cb[:2], cand(8, 2)[6:8])
    np.testing.assert_array_equal(cb[2:5], cand(3, 3))
    np.testing.assert_array_equal(cb[5:10], cand(8, 2)[3:8])    # rows past 2 + 3 keep their values
    # step 4: commit only, 2 of 3 accepted -> rows 2..4 become rows 0..2, empty live record
    e, hdr, cb, info = ora.book_step(W, N_SPEC, hdr, cb, None, num_accepted=2, parity=0)
    assert e == 0 and info == (2, 3, 1, 0)
    assert list(hdr) == [0, 0, 3, 2]
    np.testing.assert_array_equal(cb[:3], cand(3, 3))            # window rows 2..4 = step 3's candidates
    np.testing.assert_array_equal(cb[3:10], np.concatenate([cand(3, 3)[1:3], cand(8, 2)[3:8]]))
    # step 5 after the commit: the live slot (0) holds no rows, acceptance ignored, window rows 0..2
    e, hdr, cb2, info = ora.book_step(W, N_SPEC, hdr, cb, cand(1, 5), num_accepted=6, parity=1)
    assert e == 0 and info == (0, 0, 0, 1)
    assert list(hdr) == [1 | 2, 0, 1, 0]
    np.testing.assert_array_equal(cb2[:2], cb[1:3])
    np.testing.assert_array_equal(cb2[2:3], cand(1, 5))


def test_refusals_leave_everything_unchanged(ora):
    hdr = np.zeros(4, np.uint32)
    cb = buf()
    e, hdr, cb, _ = ora.book_step(W, N_SPEC, hdr, cb, cand(8, 1), 0, parity=1)
    assert e == 0
    # the same parity again: already applied
    e2, h2, c2, _ = ora.book_step(W, N_SPEC, hdr, cb, cand(8, 2), 0, parity=1)
    assert e2 == ora.BOOK_PARITY
    np.testing.assert_array_equal(h2, hdr)
    np.testing.assert_array_equal(c2, cb)
    # acceptance beyond the 8 held rows, and a negative one
    for bad in (8, 9, -1):
        e3, h3, c3, _ = ora.book_step(W, N_SPEC, hdr, cb, cand(8, 2), bad, parity=0)
        assert e3 == ora.BOOK_ACCEPTED
        np.testing.assert_array_equal(h3, hdr)
        np.testing.assert_array_equal(c3, cb)
    # a record that claims more rows than a step can write
    bogus = hdr.copy()
    bogus[1 + (int(bogus[0]) & 1)] = N_SPEC + 2
    assert ora.book_step(W, N_SPEC, bogus, cb, cand(8, 2), 0, parity=0)[0] == ora.BOOK_ACCEPTED
    # the largest valid acceptance is accepted
    assert ora.book_step(W, N_SPEC, hdr, cb, cand(8, 2), 7, parity=0)[0] == 0
    # the fresh page's parity is 0, so a first step with parity 0 is refused
    assert ora.book_step(W, N_SPEC, np.zeros(4, np.uint32), buf(), cand(8, 1), 0, parity=0)[0] == ora.BOOK_PARITY
    # more candidates than the page holds, or a buffer too short: argument errors
    assert ora.book_step(W, N_SPEC, np.zeros(4, np.uint32), buf(), cand(9, 1), 0, 1)[0] == ora.BOOK_ARG
    assert ora.book_step(W, N_SPEC, np.zeros(4, np.uint32), buf(ROWS - 1), cand(8, 1), 0, 1)[0] == ora.BOOK_ARG


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_window_follows_the_committed_stream(ora, seed):
    """Random runs of steps (0..8 candidates, random acceptance, commit-only
    steps among them): the window each step reads, and after a commit the
    buffer's first W-1 rows, are the last W-1 rows of the committed stream,
    built by brute force as a list: the initial window, then for every step
    its candidates 0..a with a the acceptance the next step passes."""
    rng = np.random.default_rng(seed)
    C = 3
    hdr = np.zeros(4, np.uint32)
    cb = rng.standard_normal((ROWS, C))
    stream = [cb[j].copy() for j in range(W - 1)]
    prev_cands = None
    parity = 0
    for step in range(40):
        n = int(rng.integers(0, N_SPEC + 2))
        x = rng.standard_normal((n, C)) if n else None
        acc = int(rng.integers(0, len(prev_cands))) if prev_cands is not None and len(prev_cands) else \
            int(rng.integers(0, 8))
        parity ^= 1
        before = cb.copy()
        e, hdr, cb, (a, n_replay, rslot, wslot) = ora.book_step(W, N_SPEC, hdr, cb, x, acc, parity)
        assert e == 0
        if prev_cands is not None and len(prev_cands):
            assert a == acc and n_replay == acc + 1
            stream.extend(prev_cands[:acc + 1])
        else:
            assert a == 0 and n_replay == 0
        # the window this step read: rows a .. a+W-2 of the buffer before it
        np.testing.assert_array_equal(before[a:a + W - 1], np.stack(stream[-(W - 1):]))
        if n == 0:
            np.testing.assert_array_equal(cb[:W - 1], np.stack(stream[-(W - 1):]))
        else:
            np.testing.assert_array_equal(cb[:W - 2], np.stack(stream[-(W - 2):]))
            np.testing.assert_array_equal(cb[W - 2:W - 2 + n], x)
            np.testing.assert_array_equal(cb[W - 2 + n:], before[W - 2 + n:])
        assert wslot == 1 - rslot and (int(hdr[0]) & 1) == wslot and int(hdr[1 + wslot]) == n
        prev_cands = x


def test_replayed_slot_is_the_previous_steps_record(ora):
    """The slot a step replays is the slot the step before wrote, so the
    replayed rows are exactly the previous step's candidates 0..a: the slots
    alternate, and each step leaves the other slot's row count as it was."""
    hdr = np.zeros(4, np.uint32)
    cb = buf()
    written = None
    for step, (n, acc) in enumerate([(8, 0), (8, 2), (5, 7), (8, 4), (2, 0), (8, 1)]):
        e, h2, cb, (a, n_replay, rslot, wslot) = ora.book_step(W, N_SPEC, hdr, cb, cand(n, step), acc,
                                                               (step + 1) & 1)
        assert e == 0
        if written is not None:
            assert rslot == written
        assert int(h2[1 + rslot]) == int(hdr[1 + rslot])
        written = wslot
        hdr = h2


def test_batch_padding_and_pages_out_of_range(ora):
    hdrs = np.zeros((3, 4), np.uint32)
    cbufs = np.stack([buf(base=1000.0 * p) for p in range(3)])
    x = np.stack([cand(8, 1 + r) for r in range(4)])
    errs, h2, c2 = ora.book_batch(W, N_SPEC, hdrs, cbufs, [2, -1, 7, 0], x, [0, 0, 0, 0], [1, 1, 1, 1])
    assert errs == [0, 0, -1, 0]
    np.testing.assert_array_equal(h2[1], hdrs[1])
    np.testing.assert_array_equal(c2[1], cbufs[1])          # no request uses page 1
    np.testing.assert_array_equal(c2[2][2:10], cand(8, 1))  # request 0 on page 2
    np.testing.assert_array_equal(c2[0][2:10], cand(8, 4))  # request 3 on page 0
