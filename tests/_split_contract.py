"""The split-KV schedule as the library's header defines it, and the checks that
any valid schedule must pass.

The pages give no balancing rule for splitting the cache (they show fixed
partition sizes for Append Attention and name FlashDecoding; PaddleNLP issue
#10157, overview; mhpq.cn article on PaddleNLP inference flags, Append
Attention), so the schedule is not part of what the method computes and the
oracle does not model it. What the decode result needs from a schedule is
that it is valid: every tile of every sequence in exactly one work unit, the
pieces of a sequence in consecutive units with their partial slots numbered
in order, and the metadata words that the kernels read agreeing with the
lengths. `check_metadata` checks exactly that on metadata read back from the
device, for any rule; `split_schedule` is the library's own rule (its
definition in include/mla_decode.h) for the word-for-word contract test.
"""
from __future__ import annotations

PAGE_TOKENS = 64
MAGIC = 0x4D4C4132
HEADER = 8


def tiles_per_sequence(seqlens):
    return [(max(int(x), 0) + PAGE_TOKENS - 1) // PAGE_TOKENS for x in seqlens]


def unpack_metadata(md, batch, units):
    """Split the int32 metadata words into named arrays (layout of the header)."""
    md = [int(x) for x in md]
    B, U = batch, units
    base = HEADER + 2 * (B + 1)
    return dict(
        magic=md[0], batch=md[1], units=md[2], units_cut=md[3], total_partials=md[4],
        units_used=md[5], seq_cost=md[6], max_pieces=md[7],
        prefix=md[HEADER:HEADER + B + 1],
        split_offset=md[HEADER + B + 1:HEADER + 2 * B + 2],
        unit_first_seq=md[base:base + U],
        unit_begin=md[base + U:base + 2 * U + 1],
        seq_first_unit=md[base + 2 * U + 1:base + 2 * U + 1 + B],
    )


def check_metadata(md, seqlens, units, min_tiles_per_unit, seq_cost):
    """Schedule-independent validity of device metadata. Raises AssertionError.

    Checks: the header names this batch and unit count; the tile prefix is the
    running sum of ceil(L_b / 64); unit ranges are contiguous, non-decreasing
    and cover [0, T) once; each non-empty unit's first sequence holds its first
    tile; each sequence with tiles has its first tile in unit seq_first_unit[b]
    and its tiles in consecutive non-empty units, as many as it has partials;
    split_offset is the running sum of those counts; units_used counts the
    non-empty units; every unit's weighted cost (tiles plus seq_cost per
    sequence start it holds) is at most ceil(W / U') + seq_cost, with W the
    weighted length and U' = md's units_cut, which is at least
    min(units, floor(W / min_tiles)) and at most units.
    """
    B, U = len(seqlens), int(units)
    m = unpack_metadata(md, B, U)
    assert m["magic"] == MAGIC, hex(m["magic"])
    assert m["batch"] == B and m["units"] == U
    T_b = tiles_per_sequence(seqlens)
    prefix = [0]
    for t in T_b:
        prefix.append(prefix[-1] + t)
    T = prefix[-1]
    assert m["prefix"] == prefix, "tile prefix"

    ub = m["unit_begin"]
    assert ub[0] == 0 and ub[U] == T, (ub[0], ub[U], T)
    assert all(ub[u] <= ub[u + 1] for u in range(U)), "unit ranges must be non-decreasing"
    owner = [None] * T
    for u in range(U):
        for f in range(ub[u], ub[u + 1]):
            assert owner[f] is None
            owner[f] = u
    assert all(o is not None for o in owner), "every tile in exactly one unit"

    def seq_of(f):
        return max(b for b in range(B) if prefix[b] <= f and T_b[b] > 0)

    nonempty = [u for u in range(U) if ub[u] < ub[u + 1]]
    assert m["units_used"] == len(nonempty)
    for u in nonempty:
        assert m["unit_first_seq"][u] == seq_of(ub[u]), f"unit {u} first sequence"

    offs = [0]
    for b in range(B):
        if T_b[b] == 0:
            offs.append(offs[-1])
            continue
        units_b = sorted(set(owner[prefix[b]:prefix[b + 1]]))
        first = m["seq_first_unit"][b]
        assert owner[prefix[b]] == first, f"sequence {b} first unit"
        # consecutive units: the piece in unit u writes partial slot
        # split_offset[b] + (u - first), so no unit may be skipped
        assert units_b == list(range(first, first + len(units_b))), f"sequence {b} units {units_b}"
        offs.append(offs[-1] + len(units_b))
    assert m["split_offset"] == offs, "split offsets"
    assert m["total_partials"] == offs[-1]
    assert m["max_pieces"] == max([offs[b + 1] - offs[b] for b in range(B)] + [0]), "largest partial count"


    c = int(seq_cost)
    assert m["seq_cost"] == c
    W = sum(t + c for t in T_b if t)
    ucut = m["units_cut"]
    mt = max(int(min_tiles_per_unit), 1)
    assert 1 <= ucut <= max(U, 1)
    assert ucut >= min(U, W // mt), (ucut, U, W, mt)
    if W:
        starts = {prefix[b] for b in range(B) if T_b[b]}
        bound = -(-W // ucut) + c
        for u in nonempty:
            cost = (ub[u + 1] - ub[u]) + c * sum(1 for f in range(ub[u], ub[u + 1]) if f in starts)
            assert cost <= bound, f"unit {u} cost {cost} > {bound}"
    return m


def split_schedule(seqlens, num_units, min_tiles_per_unit=8, seq_cost=3):
    """The library's rule, as include/mla_decode.h states it.

    T_b = ceil(L_b / 64) tiles per sequence, prefix[b] = sum of T before b,
    T = prefix[B]. On a weighted line, a sequence with tiles occupies
    seq_cost + T_b positions (its start cost, then its tiles), from
    wpre[b] = sum over b' < b of (seq_cost + T_b' if T_b' else 0); W is the
    total. With U' = max(1, min(num_units, floor(W / max(min_tiles, 1)))), the
    line is cut at cut[u] = floor(u * W / U') for u = 0..U'. Unit u < U'
    starts at the flattened tile its cut names: the tile at that position, or
    the sequence's first tile when the cut falls in the start cost; unit u
    covers tiles [unit_begin[u], unit_begin[u + 1]) and may be empty; units
    u >= U' start at T and are empty.

    Returns a dict with the metadata fields (plain Python ints/lists).
    """
    L = [max(int(x), 0) for x in seqlens]
    B = len(L)
    T_b = tiles_per_sequence(L)
    prefix = [0]
    wpre = [0]
    for t in T_b:
        prefix.append(prefix[-1] + t)
        wpre.append(wpre[-1] + (seq_cost + t if t else 0))
    T, W = prefix[-1], wpre[-1]
    units = max(int(num_units), 1)
    ucut = max(1, min(units, W // max(int(min_tiles_per_unit), 1)))

    def tile_at(v):
        if v >= W:
            return T
        b = max(i for i in range(B) if wpre[i] <= v and T_b[i] > 0)
        return prefix[b] + max(0, v - wpre[b] - seq_cost)

    unit_begin = [tile_at(u * W // ucut) if (u < ucut and W > 0) else T for u in range(units + 1)]

    def holder(f):   # the unit whose range holds tile f
        return max(u for u in range(units) if unit_begin[u] <= f)

    unit_first_seq = []
    for u in range(units):
        f = unit_begin[u]
        unit_first_seq.append(B if f >= T else max(i for i in range(B) if prefix[i] <= f))
    num_splits, seq_first_unit = [], []
    for b, t in enumerate(T_b):
        if t == 0:
            num_splits.append(0)
            seq_first_unit.append(0)
        else:
            first = holder(prefix[b])
            num_splits.append(holder(prefix[b] + t - 1) - first + 1)
            seq_first_unit.append(first)
    split_offset = [0]
    for k in num_splits:
        split_offset.append(split_offset[-1] + k)
    units_used = sum(1 for u in range(units) if unit_begin[u] < unit_begin[u + 1])
    return dict(units_cut=ucut, units_used=units_used, prefix=prefix, num_splits=num_splits,
                split_offset=split_offset, total_partials=split_offset[-1], unit_begin=unit_begin,
                unit_first_seq=unit_first_seq, seq_first_unit=seq_first_unit)


def schedule_words(seqlens, num_units, min_tiles_per_unit, seq_cost):
    """The metadata words split_schedule's result would be written as."""
    s = split_schedule(seqlens, num_units, min_tiles_per_unit, seq_cost)
    B = len(seqlens)
    return ([MAGIC, B, int(num_units), s["units_cut"], s["total_partials"], s["units_used"], seq_cost,
             max(s["num_splits"] + [0])]
            + s["prefix"] + s["split_offset"] + s["unit_first_seq"] + s["unit_begin"] + s["seq_first_unit"])
