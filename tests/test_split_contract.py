"""The split-schedule helpers of tests/_split_contract.py, on the CPU.

The library's rule (split_schedule, the header's definition) is checked
against a brute-force walk over its cut points, and the schedule-independent
validity checker (check_metadata) is checked to accept that rule's words and
to reject schedules with each kind of mistake a scheduler could make.
"""
import random

import numpy as np
import pytest

from _split_contract import check_metadata, schedule_words, split_schedule, tiles_per_sequence, HEADER


def _walk_schedule(seqlens, num_units, min_tiles, seq_cost=3):
    """Brute force: lay the sequences on a weighted line tile by tile (each
    sequence with tiles first takes seq_cost empty positions), list the cut
    points, and give every tile to the last unit whose cut is at or before
    its position."""
    T_b = [-(-max(int(x), 0) // 64) for x in seqlens]
    W = sum(t + seq_cost for t in T_b if t)
    ucut = max(1, min(num_units, W // max(min_tiles, 1)))
    cuts = [u * W // ucut for u in range(ucut)]
    owner = []   # unit of each flattened tile
    pos = 0
    for t in T_b:
        if t:
            pos += seq_cost
        for _ in range(t):
            owner.append(max(u for u in range(ucut) if cuts[u] <= pos))
            pos += 1
    assert pos == W
    pieces = {}
    f = 0
    for b, t in enumerate(T_b):
        pieces[b] = sorted(set(owner[f:f + t]))
        f += t
    # a unit starts at its first tile; units without tiles start where the
    # next tile owned by a later unit is (or at T)
    begin = [next((i for i, o in enumerate(owner) if o >= u), len(owner)) for u in range(num_units + 1)]
    return ucut, pieces, begin, owner


CASES = [
    ([256], 256, 8, 3), ([4096] * 7, 16, 8, 3), ([1, 63, 64, 65, 0, 700], 5, 1, 1),
    ([0, 0], 4, 8, 3), ([65536, 512, 3000, 70], 64, 8, 3), ([130] * 3, 1000, 1, 1),
    ([0, 512, 0, 0, 9000, 64, 0], 12, 1, 3), ([700] * 40 + [65536], 128, 8, 3),
    ([2500] * 64, 256, 8, 1), ([3000, 1, 1, 1, 5000], 7, 2, 1),
]


@pytest.mark.parametrize("seqlens,units,mt,cost", CASES)
def test_split_schedule_matches_walk(seqlens, units, mt, cost):
    sch = split_schedule(seqlens, units, mt, cost)
    ucut, pieces, begin, owner = _walk_schedule(seqlens, units, mt, cost)
    assert sch["units_cut"] == ucut
    assert sch["unit_begin"] == begin
    for b in range(len(seqlens)):
        assert sch["num_splits"][b] == len(pieces[b])
        if pieces[b]:
            assert sch["seq_first_unit"][b] == pieces[b][0]
            # pieces of a sequence sit in consecutive units
            assert pieces[b] == list(range(pieces[b][0], pieces[b][-1] + 1))
    assert sch["total_partials"] == sum(len(p) for p in pieces.values())
    assert sch["units_used"] == len(set(owner))
    assert max(owner, default=0) < units


def test_split_schedule_balances_sequence_starts():
    # many short sequences and one long one: with the start cost charged, every
    # unit's cost (tiles + 3 per sequence start in it) is within one start of
    # W / units, and every unit holds work
    seqlens = [600] * 30 + [65536]
    sch = split_schedule(seqlens, 64, 1, 3)
    T_b = [-(-x // 64) for x in seqlens]
    W = sum(t + 3 for t in T_b)
    ub = sch["unit_begin"]
    starts = set(sch["prefix"][b] for b in range(len(seqlens)) if T_b[b])
    for u in range(64):
        cost = (ub[u + 1] - ub[u]) + 3 * sum(1 for f in starts if ub[u] <= f < ub[u + 1])
        assert cost <= -(-W // 64) + 3
    assert sch["units_used"] == 64


def _random_cases(n, seed):
    rng = random.Random(seed)
    for _ in range(n):
        B = rng.choice([1, 2, 5, 17, 64])
        lens = [rng.choice([0, 1, 63, 64, 65, rng.randrange(1, 9000)]) for _ in range(B)]
        yield lens, rng.choice([1, 2, 3, 8, 13, 64, 256, 600]), rng.choice([1, 2, 8, 40]), rng.choice([1, 3])


@pytest.mark.parametrize("seqlens,units,mt,cost", CASES + list(_random_cases(40, 7)))
def test_checker_accepts_the_library_rule(seqlens, units, mt, cost):
    check_metadata(schedule_words(seqlens, units, mt, cost), seqlens, units, mt, cost)


def test_checker_accepts_another_valid_rule():
    """A different, equally valid rule (one unit per sequence, in order, the
    rest empty at the end) passes: the checker does not pin one balance."""
    lens = [700, 0, 64, 3000]
    T_b = tiles_per_sequence(lens)
    B, U = len(lens), 8
    prefix = list(np.concatenate([[0], np.cumsum(T_b)]).astype(int))
    T = prefix[-1]
    live = [b for b in range(B) if T_b[b]]
    unit_begin = [prefix[b] for b in live] + [T] * (U + 1 - len(live))
    unit_first_seq = live + [B] * (U - len(live))
    seq_first_unit, offs = [], [0]
    for b in range(B):
        seq_first_unit.append(live.index(b) if T_b[b] else 0)
        offs.append(offs[-1] + (1 if T_b[b] else 0))
    W = sum(t + 3 for t in T_b if t)
    # one sequence per unit is valid, but its balance is not within the
    # library's bound unless the cut count says so: give the largest piece's
    # cost as the bound by claiming one cut
    words = ([0x4D4C4132, B, U, 1, offs[-1], len(live), 3, 1] + prefix + offs + unit_first_seq + unit_begin
             + seq_first_unit)
    check_metadata(words, lens, U, W, 3)


def _mutations(words, B, U):
    """Each kind of scheduler mistake, as a copy of valid words."""
    base = HEADER + 2 * (B + 1)
    ub0, fsu0, so0 = base + U, base + 2 * U + 1, HEADER + B + 1

    def m(fn):
        w = list(words)
        fn(w)
        return w
    yield "magic", m(lambda w: w.__setitem__(0, 0))
    yield "prefix off by one", m(lambda w: w.__setitem__(HEADER + 1, w[HEADER + 1] + 1))
    yield "unit range overlaps", m(lambda w: w.__setitem__(ub0 + 2, w[ub0 + 1] - 1))
    yield "last unit stops short", m(lambda w: w.__setitem__(ub0 + U, w[ub0 + U] - 1))
    yield "split offset wrong", m(lambda w: w.__setitem__(so0 + B, w[so0 + B] + 1))
    yield "first unit wrong", m(lambda w: w.__setitem__(fsu0 + 1, w[fsu0 + 1] + 1))
    yield "unit first sequence wrong", m(lambda w: w.__setitem__(base + 1, w[base + 1] + 1))
    yield "units used wrong", m(lambda w: w.__setitem__(5, w[5] - 1))
    yield "largest partial count wrong", m(lambda w: w.__setitem__(7, w[7] - 1))


def test_checker_rejects_broken_schedules():
    lens = [700, 300, 64, 3000, 129]
    U = 6
    words = schedule_words(lens, U, 1, 3)
    check_metadata(words, lens, U, 1, 3)
    for what, bad in _mutations(words, len(lens), U):
        with pytest.raises(AssertionError):
            check_metadata(bad, lens, U, 1, 3)
            pytest.fail(what)


def test_checker_rejects_a_skipped_unit_inside_a_sequence():
    # sequence 0 cut over units 0 and 2 with unit 1 empty in between: its
    # second piece would write partial slot 2 of a sequence with 2 partials
    lens = [640]
    words = schedule_words(lens, 3, 1, 3)
    B, U = 1, 3
    base = HEADER + 2 * (B + 1)
    ub = words[base + U:base + 2 * U + 1]
    assert ub[0] == 0 and ub[1] < ub[2] < ub[3]
    bad = list(words)
    bad[base + U + 2] = ub[1]          # unit 1 empty, unit 2 takes its tiles
    with pytest.raises(AssertionError):
        check_metadata(bad, lens, U, 1, 3)


def test_checker_rejects_an_unbalanced_cut():
    lens = [6400]
    U = 4
    words = schedule_words(lens, U, 1, 3)
    base = HEADER + 2 * 3
    bad = list(words)
    bad[base + U + 1] = 45          # unit 0 takes 45 of 100 tiles (bound 29)
    with pytest.raises(AssertionError):
        check_metadata(bad, lens, U, 1, 3)
