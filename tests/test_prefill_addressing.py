"""Host model of the prefill kernel's addressing (prefill_mfma.hip, with the unit plan
of work_plan.hpp, the span / slot functions of device_common.hpp and the merge of
split_merge.hpp), restated in NumPy and checked on the CPU: every global offset a
thread forms (K/V tile loads through the cache's slot mapping, Q rows, output rows,
partials and their merge) lies inside its buffer as the library sizes it, every LDS
offset (staging stores, the K operand reads, the transposed V reads, the in-pool
bytes) inside its array, and each staging register slot holds the tile that the
loop stores from it.

It runs for every (waves, 16-row tiles per wave, tiles in flight) setting the build
knobs describe, including the one that faulted the GPU once (four waves of 16 rows,
four tiles in flight, on the token-major ring prefill case with 26 workgroups), over
the reduced prefill cases (ring with the sink/window mask, contiguous, paged with
its page table, head_dim 64) in both layouts, at several grid sizes and unit lengths.
Every address is in bounds in all of them; the four-tile setting instead stages the
wrong tiles (the loop alternates two register slots), a data error that the source
rules out with its static_assert."""
import numpy as np
import pytest

from kv_cache_attention_amd import workloads

TILE = 32
MIN_CHUNK_MFMA = 512                         # kvattn.cpp: units of the matrix-core kernels
UNITS_PER_WG, TAIL_PCT, TAIL_UNITS = 1, 0, 2  # kvattn.cpp defaults
SETTINGS = [(8, 2, 1), (8, 2, 2), (4, 1, 1), (4, 1, 2), (4, 1, 4)]  # waves, PF_RW, PF_AHEAD
CASES = workloads.small_prefill_variants()


class Geo:
    """Constants of one kernel instance (prefill_mfma.hip)."""

    def __init__(self, d, waves, rw, ahead):
        self.d, self.waves, self.rw, self.ahead = d, waves, rw, ahead
        self.threads = waves * 64
        self.rows = waves * rw * 16              # PF_ROWS: rows per segment
        self.ks, self.dt16 = d // 32, d // 16
        self.cpr = d * 2 // 16                   # 16-byte chunks per row
        self.krow, self.vrow = d * 2 + 16, d * 2 + 32
        self.tch = TILE * self.cpr
        assert (2 * self.tch) % self.threads == 0
        self.nch = 2 * self.tch // self.threads  # chunks per thread per tile


def host_params(case, layout, geo, inp, grid, forced):
    """The decode parameters the host fills in (kvattn.cpp fill_params / plan_for), and
    the element counts of the buffers the caller and the library allocate."""
    hkv, d = case.num_kv_heads, case.head_dim
    group = case.num_q_heads // hkv
    paged = case.cache_mode == "paged"
    unit = case.block_size if paged else case.capacity
    if layout == "token_major":
        stride_tok, stride_head = hkv * d, d
    else:
        stride_tok, stride_head = d, unit * d
    rows = case.q_len * group
    row_blocks = -(-rows // geo.rows)
    p = dict(batch=case.batch, hkv=hkv, hq=case.num_q_heads, d=d, group=group,
             q_len=case.q_len, rows=rows, cache=case.cache_mode, mask=case.mask_mode,
             n_sink=case.n_sink if case.mask_mode == "sink_window" else 0,
             window=case.window if case.mask_mode == "sink_window" else 0,
             capacity=case.capacity, stride_seq=unit * hkv * d, stride_head=stride_head,
             stride_tok=stride_tok, row_blocks=row_blocks, segs=hkv * row_blocks,
             seg_rows=geo.rows, min_chunk=forced or MIN_CHUNK_MFMA,
             upw=(1 << 30) if forced else UNITS_PER_WG, tail_pct=0 if forced else TAIL_PCT,
             seq_lens=[int(x) for x in inp["seq_lens"]],
             block_table=inp["block_table"].numpy() if paged else None,
             log2_block=int(np.log2(case.block_size)) if paged else 0,
             num_blocks=case.num_blocks if paged else 0)
    # plan_for: the step's unit bound and the workspace rows it must fit
    if case.mask_mode == "sink_window":
        n_att = min(p["n_sink"] + p["window"] + case.q_len - 1, case.capacity)
    else:
        n_att = case.capacity
    w_max = case.batch * p["segs"] * max(n_att, 1)
    units_max = -(-w_max // p["min_chunk"])
    g = min(grid, units_max)
    units = units_max if forced else min(units_max + 1, g * (UNITS_PER_WG + (TAIL_UNITS if TAIL_PCT else 0)) + 1)
    need_rows = (units + case.batch * p["segs"]) * geo.rows
    n_slots_cache = (case.num_blocks if paged else case.batch) * unit * hkv * d
    sizes = dict(cache=n_slots_cache, q=case.batch * case.q_len * case.num_q_heads * d,
                 ws_acc=need_rows * d, ws_ml=need_rows * 2, counters=case.batch * p["segs"])
    return p, max(g, 1), sizes


def seq_span(p, b):
    T = max(p["seq_lens"][b], 0)
    if p["cache"] != "ring":
        T = min(T, p["capacity"])
    sink = tail = 0
    if p["mask"] == "sink_window":
        sk = min(p["n_sink"], T)
        w0 = max(T - p["q_len"] - p["window"] + 1, 0)
        if w0 > sk:
            sink, tail = sk, w0
    s = dict(T=T, sink=sink, tail=tail, count=sink + T - tail)
    s["ring_pos0"] = max(tail, p["n_sink"])
    R = p["capacity"] - p["n_sink"]
    s["ring0"] = (s["ring_pos0"] - p["n_sink"]) % R if p["cache"] == "ring" and R > 0 else 0
    return s


def span_pos(s, j):
    return np.where(j < s["sink"], j, s["tail"] + (j - s["sink"]))


def locate(p, s, b, pos):
    """(unit, slot) of positions pos; unit -1 for a page outside the pool."""
    if p["cache"] == "contiguous":
        return np.full_like(pos, b), pos
    if p["cache"] == "ring":
        R = p["capacity"] - p["n_sink"]
        r = s["ring0"] + (pos - s["ring_pos0"])
        r = np.where(r >= R, r - R, r)
        return np.full_like(pos, b), np.where(pos < p["n_sink"], pos, p["n_sink"] + r)
    blk = p["block_table"][b, pos >> p["log2_block"]]
    ok = (blk >= 0) & (blk < p["num_blocks"])
    return np.where(ok, blk, -1), pos & ((1 << p["log2_block"]) - 1)


def plan(p, n_wg):
    """plan_flat + unit_begin: the units' flat ranges."""
    counts = [seq_span(p, b)["count"] for b in range(p["batch"])]
    total = sum(counts) * p["segs"]
    units = n_wg * p["upw"]
    usz = max(-(-total // units), p["min_chunk"])
    usz = (usz + 15) & ~15
    n_big = -(-total // usz)
    begin = lambda u: min(u * usz, total)
    unit_of = lambda x: x // usz
    return n_big, begin, unit_of, counts, total


def pieces(p, n_wg):
    """Every piece of every unit (for_each_piece_ahead), with its workspace slot."""
    n_units, begin, unit_of, counts, total = plan(p, n_wg)
    out = []
    seg0 = 0
    for b, c in enumerate(counts):
        for seg in range(p["segs"]):
            if c:
                first, last = unit_of(seg0), unit_of(seg0 + c - 1)
                for u in range(first, last + 1):
                    ja = max(begin(u), seg0) - seg0
                    jb = min(begin(u + 1), seg0 + c) - seg0
                    out.append(dict(b=b, seg=seg, ja=ja, jb=jb, unit=b * p["segs"] + seg,
                                    slot0=first + b * p["segs"] + seg, nparts=last - first + 1,
                                    part=u - first))
            seg0 += c
    assert seg0 == total
    return out, n_units


def check_piece(p, geo, pc, sizes, bad):
    d, s = p["d"], seq_span(p, pc["b"])
    b, kvh = pc["b"], pc["seg"] // p["row_blocks"]
    row0 = (pc["seg"] - kvh * p["row_blocks"]) * geo.rows
    j0, j1 = pc["ja"], pc["jb"]
    n_tiles = -(-(j1 - j0) // TILE)

    def need(name, lo, hi, limit):
        if lo < 0 or hi > limit:
            bad.append((name, int(lo), int(hi), int(limit), dict(pc)))

    # K/V tile loads: tiles 0 .. n_tiles - 1 + PF_AHEAD are issued (the ring runs ahead)
    t = np.arange(n_tiles + geo.ahead)[:, None, None]
    tid = np.arange(geo.threads)[None, :, None]
    k = np.arange(geo.nch)[None, None, :]
    cc = tid + k * geo.threads
    kind, rem = cc // geo.tch, cc % geo.tch
    j = np.minimum(j0 + t * TILE + rem // geo.cpr, j1 - 1)
    pos = span_pos(s, j)
    need("position", pos.min(), pos.max() + 1, s["T"])
    unit, idx = locate(p, s, b, pos)
    # the slot stays inside its sequence (contiguous, ring) or block (paged)
    need("slot", idx.min(), idx.max() + 1,
         p["capacity"] if p["cache"] != "paged" else 1 << p["log2_block"])
    unit = np.where(unit >= 0, unit, 0)  # out-of-pool entries read block 0
    off = (unit * p["stride_seq"] + kvh * p["stride_head"] + idx * p["stride_tok"] +
           (rem % geo.cpr) * 8)
    need("K/V load (elements)", off.min(), off.max() + 8, sizes["cache"])
    # staging stores into LDS (bytes), and the in-pool bytes (paged)
    dst = np.where(kind == 1, (rem // geo.cpr) * geo.vrow, (rem // geo.cpr) * geo.krow) + \
        (rem % geo.cpr) * 16
    need("K LDS store", dst[kind == 0].min(), dst[kind == 0].max() + 16, TILE * geo.krow)
    if (kind == 1).any():
        need("V LDS store", dst[kind == 1].min(), dst[kind == 1].max() + 16, TILE * geo.vrow)
    need("in-pool byte", 0, (rem // geo.cpr).max() + 1, TILE)

    # operand reads from LDS: K in the A layout, V through the transposed read
    lane = np.arange(64)
    lr, lq = lane % 16, lane // 16
    kr = [(tt * 16 + lr) * geo.krow + (ks * 32 + lq * 8) * 2 for tt in range(2)
          for ks in range(geo.ks)]
    need("K operand read", min(x.min() for x in kr), max(x.max() for x in kr) + 16,
         TILE * geo.krow)
    vrow0 = (lq * 4 + lr // 4) * geo.vrow + (lr % 4) * 8
    vr = [vrow0 + dt * 32 + h * 16 * geo.vrow for dt in range(geo.dt16) for h in range(2)]
    need("V transposed read", min(x.min() for x in vr), max(x.max() for x in vr) + 8,
         TILE * geo.vrow)
    need("in-pool word read", 0, 16 + 3 * 4 + 4, TILE)

    # Q rows and output rows of the waves; partials of a split segment and their merge
    wave = np.arange(geo.waves)[:, None, None]
    qt = np.arange(geo.rw)[None, :, None]
    n = row0 + wave * geo.rw * 16 + qt * 16 + lr[None, None, :]
    live = n < p["rows"]
    i = np.where(live, n // p["group"], 0)
    h = kvh * p["group"] + np.where(live, n - i * p["group"], 0)
    rid = (b * p["q_len"] + i) * p["hq"] + h
    need("Q load", (rid * d).min(), (rid * d).max() + (geo.ks * 4 - 1) * 8 + 8, sizes["q"])
    if live.any():
        need("output row", (rid[live] * d).min(), (rid[live] * d).max() + d, sizes["q"])
    if pc["nparts"] > 1:
        nb = (n - row0)[live]
        part = (pc["slot0"] + pc["part"]) * geo.rows + nb
        need("partial acc", part.min() * d, part.max() * d + d, sizes["ws_acc"])
        need("partial (m, l)", part.min() * 2, part.max() * 2 + 2, sizes["ws_ml"])
        need("arrival counter", pc["unit"], pc["unit"] + 1, sizes["counters"])
        # merge_partials, 64 rows at a time: partial k of row r at (slot0 + k) * seg_rows + r
        for r0 in range(0, geo.rows, 64):
            if row0 + r0 >= p["rows"]:
                break
            r = np.arange(64)
            r = r[row0 + r0 + r < p["rows"]]
            pk = (pc["slot0"] + np.arange(pc["nparts"]))[:, None] * p["seg_rows"] + r0 + r[None, :]
            need("merge acc read", pk.min() * d, pk.max() * d + d, sizes["ws_acc"])
            need("merge (m, l) read", pk.min() * 2, pk.max() * 2 + 2, sizes["ws_ml"])
    return n_tiles


def staging_mismatches(ahead, n_tiles):
    """The tile loop (unrolled by two: register slots 0 and 1 % ahead alternate as the
    slot being refilled and the slot stored next): tiles whose LDS buffer does not
    receive that tile's loads."""
    slot = {a: a for a in range(ahead)}  # slot -> tile whose loads it holds
    buf = {0: slot[0]}
    wrong = []
    for t in range(n_tiles):
        mine, nxt = (0, 1 % ahead) if t % 2 == 0 else (1 % ahead, 0)
        if buf[t % 2] != t:
            wrong.append(t)
        slot[mine] = t + ahead
        if t + 1 < n_tiles:
            buf[(t + 1) % 2] = slot[nxt]
    return wrong


def _model(name, layout, setting, grid, forced):
    case = CASES[name]
    geo = Geo(case.head_dim, *setting)
    inp = workloads.make_inputs(case)
    p, g, sizes = host_params(case, layout, geo, inp, grid, forced)
    pcs, n_units = pieces(p, g)
    slots = [pc["slot0"] + pc["part"] for pc in pcs]
    assert len(set(slots)) == len(slots), "one workspace slot per piece"
    bad, tiles = [], []
    for pc in pcs:
        tiles.append(check_piece(p, geo, pc, sizes, bad))
    return bad, tiles


@pytest.mark.parametrize("forced", [0, 64, 320])
@pytest.mark.parametrize("grid", [1, 26, 256])
@pytest.mark.parametrize("layout", ["token_major", "head_major"])
@pytest.mark.parametrize("setting", SETTINGS, ids=lambda s: "w%dr%da%d" % s)
@pytest.mark.parametrize("name", list(CASES))
def test_every_prefill_address_is_in_bounds(name, setting, layout, grid, forced):
    bad, _ = _model(name, layout, setting, grid, forced)
    assert not bad, bad[:5]


@pytest.mark.parametrize("setting", SETTINGS, ids=lambda s: "w%dr%da%d" % s)
def test_each_staged_tile_reaches_its_buffer(setting):
    """Two tiles in flight or fewer: every tile the loop computes is the one stored into
    its buffer.  Four in flight (a setting the source refuses): the loop's two
    alternating register slots hand later tiles' loads to the stores."""
    wrong = [staging_mismatches(setting[2], n) for n in range(1, 40)]
    if setting[2] <= 2:
        assert not any(wrong)
    else:
        assert all(w == list(range(2, n)) for w, n in zip(wrong, range(1, 40)))


def test_faulting_launch_shape_is_reproduced_by_the_model():
    """The launch recorded with the fault: ring prefill case, token-major, four waves of
    16 rows, 26 workgroups; the model has its pieces and finds no address outside a
    buffer."""
    bad, tiles = _model("prefill_ring", "token_major", (4, 1, 4), 26, 0)
    assert not bad
    assert sum(tiles) > 0


def test_model_catches_a_planted_slot_mistake():
    """The model is not vacuous: a ring slot mapping that forgets the wrap (position
    past the rolling slots) is reported."""
    case = CASES["prefill_ring"]
    geo = Geo(case.head_dim, 8, 2, 2)
    inp = workloads.make_inputs(case)
    p, g, sizes = host_params(case, "token_major", geo, inp, 26, 0)
    global locate
    orig = locate

    def no_wrap(p_, s, b, pos):
        unit, idx = orig(p_, s, b, pos)
        if p_["cache"] == "ring":
            idx = np.where(pos < p_["n_sink"], pos, p_["n_sink"] + s["ring0"] + (pos - s["ring_pos0"]))
        return unit, idx
    locate = no_wrap
    try:
        bad = []
        for pc in pieces(p, g)[0]:
            check_piece(p, geo, pc, sizes, bad)
    finally:
        locate = orig
    assert any(x[0] == "slot" for x in bad)
