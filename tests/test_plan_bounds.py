"""The unit plan's arithmetic (work_plan.hpp: plan_flat, unit_begin, unit_of and the
piece slots of for_each_piece_ahead) restated on the host, checked against the
bound the library sizes its workspace by (kvattn.cpp: plan_for).  A plan with more
slots than that bound would write past the workspace, so the bound is checked here
over many shapes and every tail setting the build knobs allow in practice."""
import random

import pytest

UNITS_PER_WG, TAIL_PCT, TAIL_UNITS = 1, 0, 2  # the library's defaults
MIN_CHUNK, MIN_CHUNK_MFMA = 256, 512


def plan(total, n_wg, min_chunk, upw=UNITS_PER_WG, tail_pct=TAIL_PCT, tail_units=TAIL_UNITS):
    units = n_wg * upw  # upw = 0: units of exactly min_chunk (forced unit lengths)
    usz = max(-(-total // units) if units > 0 else 0, min_chunk)
    usz = (usz + 15) & ~15
    big, n_big, small = usz, -(-total // usz), usz
    xb = n_big * usz
    if tail_pct > 0 and units > 0 and n_big >= units:
        b = (usz * (100 - tail_pct) // 100) & ~15
        if b < min_chunk:
            b = (min_chunk + 15) & ~15
        if units * b < total:
            rest = total - units * b
            tu = n_wg * tail_units
            s = max(-(-rest // tu), min_chunk)
            big, n_big, xb, small = b, units, units * b, (s + 15) & ~15
    n_units = -(-total // big) if xb >= total else n_big + -(-(total - xb) // small)
    begin = lambda u: u * big if u < n_big else xb + (u - n_big) * small
    unit_of = lambda x: x // big if x < xb else n_big + (x - xb) // small
    return n_units, begin, unit_of


def host_units(w_max, resident, min_chunk, tail_units=TAIL_UNITS):
    """plan_for: units the workspace check allows for (not forced)."""
    units_max = -(-w_max // min_chunk)
    g = min(resident, units_max)
    return g, min(units_max + 1, g * (UNITS_PER_WG + tail_units))


def slots(counts, segs_per_seq, n_units, begin, unit_of):
    """Workspace slot of every piece (unit + segment), walking each unit's pieces."""
    seg_start = []
    x = 0
    for c in counts:
        for _ in range(segs_per_seq):
            seg_start.append((x, c))
            x += c
    total = x
    out = []
    for u in range(n_units):
        x0, x1 = begin(u), min(begin(u + 1), total)
        assert x0 < x1, "every unit holds work"
        for s, (a, c) in enumerate(seg_start):
            if c and a < x1 and a + c > x0:
                first = unit_of(a)  # the unit of the segment's first piece
                part = u - first
                assert 0 <= part <= unit_of(a + c - 1) - first
                out.append((first + s + part, u, s))  # slot0 + part, as the kernels write
    return out, total


@pytest.mark.parametrize("tail", [(0, 2), (10, 1), (15, 2), (25, 4)])
@pytest.mark.parametrize("seed", range(40))
def test_units_partition_the_range_and_fit_the_workspace(seed, tail):
    tail_pct, tail_units = tail
    rng = random.Random(seed)
    batch = rng.randint(1, 64)
    segs_per_seq = rng.choice([1, 2, 8, 32])
    cap = rng.choice([64, 1000, 4096, 32768])
    counts = [rng.randint(0, cap) for _ in range(batch)]
    if not any(counts):
        counts[0] = 1
    mc = rng.choice([MIN_CHUNK, MIN_CHUNK_MFMA])
    resident = rng.choice([1, 7, 256, 1024])
    w_max = batch * segs_per_seq * cap
    g, allowed = host_units(w_max, resident, mc, tail_units)
    n_units, begin, unit_of = plan(sum(counts) * segs_per_seq, g, mc, tail_pct=tail_pct,
                                   tail_units=tail_units)
    assert n_units <= allowed
    ps, total = slots(counts, segs_per_seq, n_units, begin, unit_of)
    assert begin(0) == 0 and begin(n_units) >= total
    assert all(begin(u) < begin(u + 1) for u in range(n_units))
    assert all(unit_of(x) == u for u in range(n_units)
               for x in (begin(u), min(begin(u + 1), total) - 1))
    sl = [p[0] for p in ps]
    assert len(set(sl)) == len(sl), "one slot per piece"
    assert max(sl) < n_units + batch * segs_per_seq


def test_tail_takes_the_requested_share():
    # 256 workgroups, decode_7b-sized work: head units cover 85 %, the rest is in
    # at most two tail units per workgroup
    total = 16 * 32 * 2560
    n_units, begin, _ = plan(total, 256, MIN_CHUNK, tail_pct=15, tail_units=2)
    head = begin(256)
    assert 0.84 <= head / total <= 0.86
    assert 256 < n_units <= 256 * 3


def test_small_work_has_no_tail():
    n_units, begin, _ = plan(1000, 256, MIN_CHUNK)
    assert n_units == 4 and begin(1) == 256


FLAT_MAX = 1 << 30  # largest flat range of one launch (device_common.hpp: kFlatMax)
INT32_MAX = (1 << 31) - 1


@pytest.mark.parametrize("seed", range(10))
def test_forced_units_are_exactly_min_chunk(seed):
    # forced unit lengths pass units_per_wg = 0: every unit but the last is min_chunk
    rng = random.Random(100 + seed)
    counts = [rng.randint(0, 5000) for _ in range(rng.randint(1, 16))]
    counts[0] += 1
    segs = rng.choice([1, 8])
    mc = rng.choice([64, 256, 1024])
    total = sum(counts) * segs
    n_units, begin, unit_of = plan(total, rng.choice([1, 64, 256]), mc, upw=0)
    assert n_units == -(-total // ((mc + 15) & ~15))
    assert all(begin(u + 1) - begin(u) == ((mc + 15) & ~15) for u in range(n_units - 1))
    ps, _ = slots(counts, segs, n_units, begin, unit_of)
    sl = [p[0] for p in ps]
    assert len(set(sl)) == len(sl) and max(sl) < n_units + len(counts) * segs


@pytest.mark.parametrize("tail", [(0, 2), (15, 2), (25, 4)])
@pytest.mark.parametrize("n_wg", [1, 2, 255, 256, 1024])
@pytest.mark.parametrize("mc", [256, 512, 1 << 24])
def test_plan_indices_fit_32_bits_up_to_the_flat_limit(tail, n_wg, mc):
    # every value the 32-bit plan forms (work_plan.hpp) stays below 2^31 for flat
    # ranges up to the per-launch limit: the sums it divides, unit boundaries up to
    # one past the last unit, and the tail's shares
    tail_pct, tail_units = tail
    for total in (1, 15, 16, FLAT_MAX // 3, FLAT_MAX - 1, FLAT_MAX):
        for upw in (UNITS_PER_WG, 0):
            units = n_wg * upw
            usz = max(-(-total // units) if units > 0 else 0, mc)
            assert total + units - 1 <= INT32_MAX
            usz = (usz + 15) & ~15
            assert total + usz - 1 <= INT32_MAX
            n_units, begin, unit_of = plan(total, n_wg, mc, upw=upw, tail_pct=tail_pct,
                                           tail_units=tail_units)
            assert max(begin(n_units), begin(n_units - 1) + usz) <= INT32_MAX
            # the last unit ends at or past the total, and unit_of inverts begin
            assert begin(n_units) >= total and unit_of(total - 1) == n_units - 1


def batch_ranges(batch, per_seq, flat_max=FLAT_MAX):
    """kvattn.cpp launch_decode: one launch, or one per batch range of at most
    flat_max // per_seq sequences (per_seq = segments x the longest attended set)."""
    if batch * per_seq <= flat_max:
        return [(0, batch)]
    per_launch = flat_max // per_seq
    assert per_launch >= 1
    return [(b0, min(per_launch, batch - b0)) for b0 in range(0, batch, per_launch)]


@pytest.mark.parametrize("batch,per_seq,flat_max", [
    (1, 1, FLAT_MAX), (4096, 8 * 131072, FLAT_MAX), (256, 16 * 1048576, FLAT_MAX),
    (7, 1000, 3000), (8, 65536, 131072), (3, 5, 5)])
def test_batch_ranges_cover_the_batch_within_the_limit(batch, per_seq, flat_max):
    rs = batch_ranges(batch, per_seq, flat_max)
    assert [b0 for b0, _ in rs] == list(range(0, batch, rs[0][1]))
    assert sum(n for _, n in rs) == batch
    assert all(n >= 1 and n * per_seq <= flat_max for _, n in rs)
