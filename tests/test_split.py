"""Host logic of the tail split: which tail tiles are cut, into which pieces, and which
workgroup runs each piece (CPU only: no call here launches a kernel).

A launch of T tiles on P units runs T // P whole rounds; the R = T % P tail tiles are cut
along the contraction (k-steps of the tile) into pieces.  The checks: every tail tile's
k-range is covered exactly once by its pieces, in piece order, on multiples of 4 k-steps;
each workgroup runs at most one piece; the modes, piece counts and workgroup deals follow
the rules stated in the library; and a per-XCD simulation of the hardware's in-order
dispatch finishes the tail well before a whole tile time."""

from __future__ import annotations

import pytest

import newton_schulz_02_amd as nm

UNIT = 4   # pieces start and end on multiples of 4 k-steps
XCDS = 8


def _coverage(plan, items, ks):
    by_tile = {}
    for it in items:
        if it is None:
            continue
        t, piece, pieces, k0, k1 = it
        by_tile.setdefault(t, []).append((piece, pieces, k0, k1))
    return by_tile


CASES = [(952, 256, 64), (672, 256, 64), (960, 256, 64), (992, 256, 64), (2105, 256, 64),
         (3088, 256, 64), (160, 256, 16), (160, 256, 64), (128, 256, 64), (1, 256, 64),
         (10, 256, 16), (10, 256, 64), (257, 256, 32), (255, 256, 64), (952, 256, 172),
         (100, 32, 64), (40, 32, 32), (7, 8, 64), (300, 256, 8), (512, 256, 64),
         (952, 256, 18), (160, 256, 18), (20, 256, 66), (200, 256, 130), (3, 256, 22)]


@pytest.mark.parametrize("tiles,units,ks", CASES)
def test_pieces_cover_every_tail_tile_once(tiles, units, ks):
    plan, items = nm.split_plan(tiles, units, ks)
    R = plan["tail"]
    assert plan["dp_tiles"] + R == tiles
    if plan["mode"] == 0:
        assert R == 0 and plan["tail_wgs"] == 0 and items == []
        return
    assert plan["dp_tiles"] % units == 0 and 0 < R < units
    assert len(items) == plan["tail_wgs"]
    by_tile = _coverage(plan, items, ks)
    assert sorted(by_tile) == list(range(R))
    real = 0
    for t, ps in by_tile.items():
        ps.sort()
        pieces = ps[0][1]
        assert [p for p, *_ in ps] == list(range(pieces)), t
        assert all(n == pieces for _, n, _, _ in ps)
        assert ps[0][2] == 0 and ps[-1][3] == ks
        for (_, _, a0, a1), (_, _, b0, _) in zip(ps, ps[1:]):
            assert a1 == b0
        for _, _, k0, k1 in ps:
            assert k0 < k1 and k0 % UNIT == 0 and (k1 % UNIT == 0 or k1 == ks)
        real += pieces
    assert real <= plan["slots"]


@pytest.mark.parametrize("tiles,units,ks", CASES)
def test_modes_and_deals(tiles, units, ks):
    plan, items = nm.split_plan(tiles, units, ks)
    R = tiles % units
    if plan["mode"] == 0:
        # Nothing to cut, contraction too short to cut, or a cut not worth it.
        assert R == 0 or ks // UNIT < 4 or 2 * R > units
        return
    if 2 * R <= units:
        c = plan["pieces_or_n"]
        assert plan["mode"] == 1 and 2 <= c <= min(8, units // R, ks // UNIT // 2)
        assert plan["tail_wgs"] == c * R and None not in items
    else:
        n = plan["pieces_or_n"]
        assert plan["mode"] == 2 and n == -(-R // (units - R))
        assert plan["tail_wgs"] % (2 * XCDS) == 0 and plan["tail_wgs"] >= 2 * R
        # Each XCD (workgroup j on XCD j % 8) gets the first pieces of a run of tiles, then
        # the second pieces of the same run.
        for x in range(XCDS):
            seq = [items[j] for j in range(x, len(items), XCDS) if items[j] is not None]
            firsts = [t for t, p, *_ in seq if p == 0]
            seconds = [t for t, p, *_ in seq if p == 1]
            assert seq[:len(firsts)] == [s for s in seq if s[1] == 0]
            assert firsts == seconds
            assert firsts == list(range(firsts[0], firsts[0] + len(firsts))) if firsts else True


def _tail_makespan(plan, items, units):
    """Per XCD, dispatch its workgroups in order to the first free unit (units // 8 per
    XCD); a piece takes k1 - k0."""
    per = max(1, units // XCDS)
    worst = 0
    for x in range(XCDS):
        free = [0] * per
        for j in range(x, len(items), XCDS):
            if items[j] is None:
                continue
            _, _, _, k0, k1 = items[j]
            u = min(range(per), key=lambda i: free[i])
            free[u] += k1 - k0
        worst = max(worst, max(free))
    return worst


@pytest.mark.parametrize("tiles,units,ks", [c for c in CASES if c[1] == 256])
def test_tail_finishes_well_before_a_whole_tile(tiles, units, ks):
    plan, items = nm.split_plan(tiles, units, ks)
    if plan["mode"] == 0:
        return
    span = _tail_makespan(plan, items, units)
    assert span <= 0.9 * ks, (plan, span)
    if plan["mode"] == 1:
        c = plan["pieces_or_n"]
        assert span <= -(-ks // c // UNIT) * UNIT + UNIT


def test_no_split_cases():
    assert nm.split_plan(512, 256, 64)[0]["mode"] == 0      # whole rounds
    assert nm.split_plan(952, 256, 12)[0]["mode"] == 0      # contraction too short
    assert nm.split_plan(250, 256, 64)[0]["mode"] == 0      # 250 of 256: a cut gains nothing
    assert nm.split_plan(0, 256, 64)[0]["mode"] == 0
    with pytest.raises(nm.MuonError):
        nm.split_plan(-1, 256, 64)


def _gemms(shapes, dtype=nm.MUON_BF16, **hp):
    d = nm.plan_describe(nm.shape_array(shapes, dtype=dtype), len(shapes), nm.make_hparams(**hp))
    return d, [L for L in d["launches"] if L["kind"] == "gemm"]


LAYER = [(4096, 4096)] * 4 + [(4096, 11008)] * 2 + [(11008, 4096)]


def test_layer_plan_splits():
    d, gemms = _gemms(LAYER)
    assert d["units"] == 256
    for L in gemms:
        for sh, tiles in enumerate(L["tiles_cfg"]):
            sp = L["split_cfg"][sh]
            ref, _ = nm.split_plan(tiles, 256, L["kmin_cfg"][sh])
            assert (sp["mode"], sp["dp_tiles"], sp["tail"], sp["tail_wgs"], sp["slots"]) == \
                (ref["mode"], ref["dp_tiles"], ref["tail"], ref["tail_wgs"], ref["slots"])
            assert sp["slots"] <= d["split_slots"]
    sym = gemms[1]   # a symmetric level: 952 square tiles, tail of 184 cut once after 48 of 64
    # (7 lower triangles of 16 x 16 square, 11 x 16 wide and 32 x 32 small tiles)
    assert sym["tiles_cfg"] == [952, 672, 3696] and sym["kmin_cfg"] == [64, 64, 64]
    assert sym["split_cfg"][0]["mode"] == 2 and sym["split_cfg"][0]["n"] == 3
    assert sym["split_cfg"][0]["tail"] == 184
    upd = gemms[-1]  # the update: 2105 wide tiles, tail of 57 cut into 4
    assert upd["tiles_cfg"][1] == 2105 and upd["split_cfg"][1]["mode"] == 1
    assert upd["split_cfg"][1]["c"] == 4
    # The Gram formation of the wide matrices contracts over 11008; its tail tiles are the
    # square matrices' (4096).
    assert gemms[0]["kmin_cfg"] == [64, 64, 64]


def test_kmin_is_the_tail_tiles_contraction():
    # fp32: 128 bytes hold 32 elements per k-step; a 1024 x 1024 Gram product has 32 k-steps.
    _, gemms = _gemms([(1024, 1024)], dtype=nm.MUON_F32)
    assert all(L["kmin_cfg"] == [32, 32, 32] for L in gemms if L["signature"].startswith("f32|2"))
    # bf16 ragged: m = 1100 pads to 1152, 18 k-steps (not a multiple of 4): at most 2 equal
    # pieces of at least 2 units, the last ending at 18.
    _, gemms = _gemms([(1100, 1500)])
    for L in gemms:
        if L["signature"].startswith("bf16|2"):
            assert L["kmin_cfg"] == [18, 18, 18]
            assert L["split_cfg"][0]["mode"] == 1 and L["split_cfg"][0]["c"] == 2


@pytest.fixture
def clean_table():
    nm.tune_clear()
    nm.tune_force(None)
    yield
    nm.tune_clear()
    nm.tune_force(None)


def test_forced_split_configurations(clean_table):
    for cfg in (nm.CFG_SQUARE_SPLIT, nm.CFG_WIDE_SPLIT):
        nm.tune_force(cfg)
        _, gemms = _gemms(LAYER)
        for L in gemms:
            sh = cfg & 1
            sp = L["split_cfg"][sh]
            if sp["mode"] == 0:
                assert L["cfg"] == sh and L["grid"] == L["tiles"]
            else:
                assert L["cfg"] == cfg and L["grid"] == sp["dp_tiles"] + sp["tail_wgs"]
            assert L["tiles"] == L["tiles_cfg"][sh]
    # A launch whose tail is too short to cut runs unsplit.
    nm.tune_force(nm.CFG_SQUARE_SPLIT)
    _, gemms = _gemms([(100, 300)])
    assert all(L["cfg"] == 0 for L in gemms)


def test_split_choices_import_and_export(clean_table):
    _, gemms = _gemms(LAYER)
    sig = gemms[1]["signature"]
    nm.tune_import(f"{sig} 2\n")
    assert nm.tune_table() == {sig: 2}
    assert nm.tune_export() == f"# muon-tune {nm.kernel_hash()}\n{sig} 2\n"
    _, gemms = _gemms(LAYER)
    assert [L["cfg"] for L in gemms if L["signature"] == sig] == [2] * sum(
        L["signature"] == sig for L in gemms)


def _regions(d, desc_bytes):
    """Every byte range [lo, hi) of the workspace the plan hands out."""
    n = d["count"]
    out = [(d["desc_off"], d["desc_off"] + n * desc_bytes), (d["scale_off"], d["scale_off"] + 4 * n),
           (d["partial_off"], d["partial_off"] + 4 * d["mom_tiles"]),
           (d["split_cnt_off"], d["split_cnt_off"] + 4 * d["split_cnt_n"]),
           (d["split_slot_off"], d["split_slot_off"] + d["split_slots"] * 256 * 384 * 4)]
    for m in d["matrices"]:
        out += [(o, o + b) for o, b in m["regions"]]
    return [r for r in out if r[1] > r[0]]


@pytest.mark.parametrize("shapes,dtype", [
    (LAYER, nm.MUON_BF16),
    ([(1024, 1024)], nm.MUON_BF16),
    ([(1100, 1500), (1500, 1100), (64, 64), (1, 1)], nm.MUON_BF16),
    ([(2048, 2048)] * 4, nm.MUON_F32),
    ([(1200, 1000)], nm.MUON_F32),
])
def test_workspace_regions_are_disjoint(shapes, dtype):
    """Descriptors, scales, partial sums, split counters and slots, and every matrix's Gram
    slots and X forms occupy disjoint ranges inside the workspace."""
    d, _ = _gemms(shapes, dtype=dtype)
    regions = sorted(_regions(d, 1))
    assert regions[0][0] >= 0 and regions[-1][1] <= d["workspace"]
    for (a0, a1), (b0, b1) in zip(regions, regions[1:]):
        assert a1 <= b0, ((a0, a1), (b0, b1))
    # The status word's 256 bytes come first, then count MatDesc entries before the scales.
    assert d["desc_off"] == 256 and d["scale_off"] > d["desc_off"]


def test_workspace_holds_the_partial_sums():
    d, _ = _gemms(LAYER)
    slot_bytes = 256 * 384 * 4
    assert d["split_slots"] >= 448 and d["split_slot_off"] + d["split_slots"] * slot_bytes <= d["workspace"]
    # The slots come after everything else: the workspace without the split (a call whose
    # launches have nothing to cut) is the same plan up to split_slot_off.
    assert d["split_cnt_off"] + 4 * d["split_cnt_n"] <= d["split_slot_off"]
    ws_no_slots = d["workspace"] - d["split_slots"] * slot_bytes
    assert d["split_slot_off"] >= ws_no_slots - 256
    assert d["split_cnt_n"] == 512 and d["split_cnt_off"] % 256 == 0
    # Small calls reserve little: one 64 x 64 matrix has no tail to cut.
    d, _ = _gemms([(64, 64)])
    assert d["split_slots"] == 0


def test_buffer_offsets_flag():
    """The 256 x 256 kernel uses 32-bit buffer offsets only while every operand of a launch is
    below 2 GB: a 32768 x 32768 bf16 matrix (2 GiB operands) turns it off for its launches."""
    hp = nm.make_hparams()
    small = nm.plan_describe(nm.shape_array([(4096, 11008)]), 1, hp)
    assert all(L["buf_ok"] for L in small["launches"] if L["kind"] == "gemm")
    big = nm.plan_describe(nm.shape_array([(32768, 32768)]), 1, hp)
    assert not any(L["buf_ok"] for L in big["launches"] if L["kind"] == "gemm")
    mixed = nm.plan_describe(nm.shape_array([(32768, 32768), (512, 512)]), 2, hp)
    assert not any(L["buf_ok"] for L in mixed["launches"] if L["kind"] == "gemm")


def test_long_fp32_contractions_always_split():
    """fp32 Gram formations over 2^17 or more elements run split whatever the configuration
    asked for (accuracy of the fp32 sums); shorter ones and bf16 ones follow the request."""
    hp = nm.make_hparams()
    try:
        nm.tune_force(nm.CFG_SQUARE)
        long = nm.plan_describe(nm.shape_array([(3, 1 << 20, nm.MUON_F32)]), 1, hp)
        syrk = long["launches"][2]
        assert syrk["groups"][0]["kind"] == "syrk" and syrk["cfg"] == nm.CFG_SQUARE_SPLIT
        assert syrk["split_cfg"][0]["mode"] == 1 and syrk["split_cfg"][0]["c"] == 8
        assert all(L["cfg"] == nm.CFG_SQUARE for L in long["launches"][3:] if L["kind"] == "gemm")
        thin_bf16 = nm.plan_describe(nm.shape_array([(3, 1 << 20, nm.MUON_BF16)]), 1, hp)
        assert thin_bf16["launches"][2]["cfg"] == nm.CFG_SQUARE_SPLIT  # fp32 Gram space (m <= 128)
        short = nm.plan_describe(nm.shape_array([(3, 1 << 16, nm.MUON_F32)]), 1, hp)
        assert all(L["cfg"] == nm.CFG_SQUARE for L in short["launches"] if L["kind"] == "gemm")
        bf16 = nm.plan_describe(nm.shape_array([(256, 1 << 20, nm.MUON_BF16)]), 1, hp)
        assert all(L["cfg"] == nm.CFG_SQUARE for L in bf16["launches"] if L["kind"] == "gemm")
        # 256 x 384 tiles are out at this length (32-bit offsets): the split runs on 256 x 256
        nm.tune_force(nm.CFG_WIDE)
        wide = nm.plan_describe(nm.shape_array([(3, 1 << 20, nm.MUON_F32)]), 1, hp)
        assert wide["launches"][2]["cfg"] == nm.CFG_SQUARE_SPLIT
    finally:
        nm.tune_force(None)


def test_long_fp32_split_cuts_only_the_tail():
    """What the long-fp32 rule guarantees, per launch: its tail tiles (all of them below one
    tile per unit) are cut -- 8 pieces for at most units/8 tail tiles, units/R pieces for R up
    to units/2, one cut beyond -- and whole-round tiles keep the whole contraction."""
    hp = nm.make_hparams()
    k = 1 << 17
    try:
        nm.tune_force(nm.CFG_SQUARE)
        for m, tiles, mode, pieces, dp in ((1024, 10, 1, 8, 0), (4096, 136, 2, 2, 0), (8192, 528, 1, 8, 512)):
            d = nm.plan_describe(nm.shape_array([(m, k, nm.MUON_F32)]), 1, hp)
            syrk = d["launches"][2]
            sp = syrk["split_cfg"][0]
            assert syrk["tiles"] == tiles and syrk["cfg"] == nm.CFG_SQUARE_SPLIT
            assert sp["mode"] == mode and sp["dp_tiles"] == dp and sp["tail"] == tiles - dp
            if mode == 1:
                assert sp["c"] == pieces
            # the longest piece of a tail tile, in k-steps of 32 fp32 elements
            ks = k // 32
            items = [it for it in nm.split_plan(tiles, 256, ks)[1] if it[0] >= 0]
            longest = max(k1 - k0 for _, _, _, k0, k1 in items)
            if mode == 1:
                assert longest * pieces <= ks + 4 * pieces    # pieces start on 4-k-step units
            else:
                assert longest < ks
    finally:
        nm.tune_force(None)
