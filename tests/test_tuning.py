"""Host logic of the shape-adaptive kernel selection: the 256 x 384 configuration's tile orders
and tile counts, launch signatures, and the tuning table (force, import, export).  CPU only:
no call here launches a kernel."""

from __future__ import annotations

import itertools

from pathlib import Path

import pytest

import newton_schulz_02_amd as nm

WM, WN = 256, 384


def cdiv(a, b):
    return -(-a // b)


def wide_sym_set(m):
    """Brute force: the 256 x 384 tiles of an m x m output that hold an element on or below
    the diagonal (row >= column)."""
    out = set()
    for i in range(cdiv(m, WM)):
        last_row = min(i * WM + WM - 1, m - 1)
        for j in range(cdiv(m, WN)):
            if last_row >= j * WN:
                out.add((i, j))
    return out


@pytest.mark.parametrize("m", [1, 100, 256, 257, 383, 384, 385, 640, 768, 1000, 1152, 4096, 11008])
def test_wide_symmetric_order_covers_the_triangle_once(m):
    order = nm.wide_tile_order(True, m)
    assert len(order) == len(set(order))
    assert set(order) == wide_sym_set(m)


@pytest.mark.parametrize("rows,cols", [(1, 1), (100, 300), (300, 100), (256, 384), (257, 385),
                                       (4096, 11008), (11008, 4096), (640, 640)])
def test_wide_full_order_is_a_bijection(rows, cols):
    order = nm.wide_tile_order(False, rows, cols)
    grid = set(itertools.product(range(cdiv(rows, WM)), range(cdiv(cols, WN))))
    assert len(order) == len(grid) and set(order) == grid


def _signature_groups(sig):
    dtype, *groups = sig.split("|")
    out = []
    for g in groups:
        kind, tri, nmflag, shapes = g.split(":", 3)
        for item in shapes.split(":"):
            shape, count = item.split("*")
            m, n = (int(x) for x in shape.split("x"))
            out.append((int(kind), int(tri), int(nmflag), m, n, int(count)))
    return dtype, out


def _expected_tiles(groups):
    sq = wide = small = 0
    for kind, tri, nmflag, m, n, count in groups:
        if tri:
            t = cdiv(m, 256)
            sq += count * t * (t + 1) // 2
            wide += count * len(wide_sym_set(m))
            t = cdiv(m, 128)
            small += count * t * (t + 1) // 2
            continue
        # Full outputs are m x n: the restart product Q X and the update (n x m for the update
        # of a transposed tall matrix).
        assert kind in (3, 4)
        rows, cols = m, n
        if nmflag:
            rows, cols = cols, rows
        sq += count * cdiv(rows, 256) * cdiv(cols, 256)
        wide += count * cdiv(rows, WM) * cdiv(cols, WN)
        small += count * cdiv(rows, 128) * cdiv(cols, 128)
    return sq, wide, small


@pytest.mark.parametrize("shapes", [
    [(300, 100), (100, 300), (640, 640)],
    [(4096, 4096)] * 4 + [(4096, 11008)] * 2 + [(11008, 4096)],
    [(1000, 700), (700, 1000), (129, 1), (1, 129), (2048, 6000)],
])
def test_tile_counts_of_every_tile_shape(shapes):
    arr = nm.shape_array(shapes)
    d = nm.plan_describe(arr, len(shapes), nm.make_hparams())
    gemms = [L for L in d["launches"] if L["kind"] == "gemm"]
    assert gemms
    for L in gemms:
        dtype, groups = _signature_groups(L["signature"])
        # The signature names the launch's operand dtype: bf16, or f32 for the Gram iteration
        # of bf16 matrices with at most 128 Gram rows.
        assert dtype == {1: "bf16", 2: "f32"}[L["dtype"]]
        assert all((m <= 128) == (dtype == "f32") for *_, m, n, c in groups)
        assert sum(c for *_, c in groups) >= 1
        assert tuple(L["tiles_cfg"]) == _expected_tiles(groups), L["signature"]
        # untuned default: 128 x 128 tiles below 64 tiles of 256 x 256, else 256 x 256
        cfg = nm.CFG_SMALL if L["tiles_cfg"][0] < 64 else nm.CFG_SQUARE
        assert L["cfg"] == cfg and L["tiles"] == L["tiles_cfg"][2 if cfg == nm.CFG_SMALL else 0]
        assert L["grid"] == L["tiles"]


def test_nm_flag_marks_the_transposed_tall_update():
    d = nm.plan_describe(nm.shape_array([(300, 200)]), 1, nm.make_hparams())
    last = [L for L in d["launches"] if L["kind"] == "gemm"][-1]
    assert last["signature"] == "bf16|4:0:1:200x300*1"
    d = nm.plan_describe(nm.shape_array([(200, 300)]), 1, nm.make_hparams())
    last = [L for L in d["launches"] if L["kind"] == "gemm"][-1]
    assert last["signature"] == "bf16|4:0:0:200x300*1"
    # A small bf16 matrix iterates (and updates) in the fp32 kernel.
    d = nm.plan_describe(nm.shape_array([(300, 100)]), 1, nm.make_hparams())
    last = [L for L in d["launches"] if L["kind"] == "gemm"][-1]
    assert last["signature"] == "f32|4:0:1:100x300*1"


def test_fp32_signatures_name_their_dtype():
    d = nm.plan_describe(nm.shape_array([(300, 200)], dtype=nm.MUON_F32), 1, nm.make_hparams())
    sigs = [L["signature"] for L in d["launches"] if L["kind"] == "gemm"]
    assert sigs and all(s.startswith("f32|") for s in sigs)


@pytest.fixture
def clean_table():
    nm.tune_clear()
    nm.tune_force(None)
    yield
    nm.tune_clear()
    nm.tune_force(None)


def _cfgs(shapes):
    d = nm.plan_describe(nm.shape_array(shapes), len(shapes), nm.make_hparams())
    return [(L["signature"], L["cfg"], L["tiles"], L["tiles_cfg"]) for L in d["launches"]
            if L["kind"] == "gemm"]


def _default(tcfg):
    return nm.CFG_SMALL if tcfg[0] < 64 else nm.CFG_SQUARE


def test_table_and_force_select_the_configuration(clean_table):
    shapes = [(640, 640), (300, 100), (4096, 4096)]
    base = _cfgs(shapes)
    # Without a table entry a launch of fewer than 64 tiles of 256 x 256 runs 128 x 128 tiles.
    assert all(c == _default(tcfg) for _, c, _, tcfg in base)
    assert {c for _, c, _, _ in base} == {nm.CFG_SQUARE, nm.CFG_SMALL}
    # One signature to the wide configuration: only launches with that signature change.
    sig = base[0][0]
    nm.tune_import(f"{sig} 1\n")
    assert nm.tune_table() == {sig: 1}
    for s, c, tiles, tcfg in _cfgs(shapes):
        assert c == (1 if s == sig else _default(tcfg))
        assert tiles == tcfg[{0: 0, 1: 1, 5: 2}[c]]
    nm.tune_force(nm.CFG_WIDE)
    assert all(c == 1 for _, c, _, _ in _cfgs(shapes))
    nm.tune_force(nm.CFG_SQUARE)
    assert all(c == 0 for _, c, _, _ in _cfgs(shapes))
    nm.tune_force(None)
    assert [c for _, c, _, _ in _cfgs(shapes)] == [1 if s == sig else _default(t) for s, _, _, t in base]


def test_forced_small_tiles(clean_table):
    """Configuration 5 runs every launch on 128 x 128 tiles, except fp32 launches whose tail
    tiles contract over 2^17 elements or more: those keep the 256 x 256 tail split."""
    shapes = [(640, 640), (300, 100), (1000, 700), (129, 1)]
    nm.tune_force(nm.CFG_SMALL)
    for s, c, tiles, tcfg in _cfgs(shapes):
        assert c == nm.CFG_SMALL and tiles == tcfg[2], s
    d = nm.plan_describe(nm.shape_array([(1024, 1 << 17, nm.MUON_F32)]), 1, nm.make_hparams())
    syrk = d["launches"][2]
    assert syrk["cfg"] == nm.CFG_SQUARE_SPLIT and syrk["tiles"] == syrk["tiles_cfg"][0]
    others = [L for L in d["launches"][3:] if L["kind"] == "gemm"]
    assert others and all(L["cfg"] == nm.CFG_SMALL for L in others)


def test_export_import_round_trip(clean_table):
    head = f"# muon-tune {nm.kernel_hash()}\n"
    assert nm.tune_export() == head
    text = "bf16|0:1:0:640x640*1 1\nbf16|4:0:1:100x300*1 0\nf32|2:1:0:64x64*3 1\n"
    nm.tune_import(text)
    out = nm.tune_export()
    assert out.startswith(head)
    body = out[len(head):]
    assert sorted(body.splitlines()) == sorted(text.splitlines())
    assert body == "".join(sorted(ln + "\n" for ln in text.splitlines()))  # sorted by signature
    nm.tune_clear()
    nm.tune_import(out)
    assert nm.tune_export() == out
    # Overwrite and blank lines.
    nm.tune_import("\nbf16|0:1:0:640x640*1 0\n\n")
    assert nm.tune_table()["bf16|0:1:0:640x640*1"] == 0


@pytest.mark.parametrize("bad", ["sig", "sig 6", "sig -1", " 1", "a b 1", "sig 1x", "sig ", "sig 12"])
def test_malformed_import_adds_nothing(clean_table, bad):
    nm.tune_import("keep 1\n")
    with pytest.raises(nm.MuonError):
        nm.tune_import(f"new 0\n{bad}\n")
    assert nm.tune_table() == {"keep": 1}


def test_argument_errors(clean_table):
    for cfg in (-2, 6, 7):
        with pytest.raises(nm.MuonError):
            nm.tune_force(cfg)
    hp = nm.make_hparams()
    for reps in (0, 65):
        with pytest.raises(nm.MuonError):
            nm.tune_raw(nm.shape_array([(64, 64)]), 1, hp, 0, 0, 0, 0, None, reps=reps)


def test_tune_scratch_size_and_checks(clean_table):
    """The copies live in caller scratch: params + momenta, each 256-byte aligned; a short,
    NULL or misaligned scratch is refused on the host (fake pointers never reach a device)."""
    hp = nm.make_hparams()
    shapes = [(64, 64), (100, 30)]
    arr = nm.shape_array(shapes)
    need = nm.tune_scratch_size_raw(arr, 2, hp)
    assert need == 2 * 8192 + 2 * 6144          # 64*64*2 = 8192; 100*30*2 = 6000 -> 6144
    assert nm.tune_scratch_size_raw(nm.shape_array([]), 0, hp) == 0
    f32 = nm.shape_array([(10, 10)], dtype=nm.MUON_F32)
    assert nm.tune_scratch_size_raw(f32, 1, hp) == 2 * 512
    ws = nm.workspace_size_raw(arr, 2, hp)
    for ptr, nbytes, status in ((0, need, -1), (1 << 30, need - 1, -2), ((1 << 30) + 16, need, -1)):
        with pytest.raises(nm.MuonError) as ei:
            nm.tune_raw(arr, 2, hp, 1 << 36, ws, ptr, nbytes, None, reps=1)
        assert ei.value.status == status


def test_wide_configuration_is_off_for_operands_beyond_32_bit_offsets(clean_table):
    """(d + 384) * round_up(d, 128) * 2 >= 2^31 for d = 32768 (bf16); d = 32000 fits."""
    nm.tune_force(nm.CFG_WIDE)
    for d, ok in ((32000, True), (32768, False)):
        shapes = [(d, d), (256, 512)]
        desc = nm.plan_describe(nm.shape_array(shapes), 2, nm.make_hparams())
        for L in desc["launches"]:
            if L["kind"] != "gemm":
                continue
            has_big = f"{d}x{d}" in L["signature"]
            assert L["wide_ok"] == (ok or not has_big)
            assert L["cfg"] == (1 if L["wide_ok"] else 0)


# ---- persistent tuning tables, versioned by the kernels they were measured on ----------------

def test_the_table_names_the_kernels_it_was_measured_on(clean_table):
    """The exported table's first line is the hash of the kernel sources the library was
    built from; that is the hash of the sources in this tree (the library is current)."""
    from newton_schulz_02_amd.build import kernel_hash

    assert nm.kernel_hash() == kernel_hash()
    assert len(nm.kernel_hash()) == 16 and int(nm.kernel_hash(), 16) >= 0
    assert nm.tune_export().splitlines()[0] == f"# muon-tune {nm.kernel_hash()}"


def test_a_table_of_other_kernels_is_refused(clean_table):
    nm.tune_import("keep 1\n")
    other = "0" * 16 if nm.kernel_hash() != "0" * 16 else "1" * 16
    with pytest.raises(nm.MuonError) as ei:
        nm.tune_import(f"# muon-tune {other}\nnew 0\n")
    assert ei.value.status == nm.MUON_ESTALE
    assert nm.tune_table() == {"keep": 1}
    # its own hash, comments and a text without the line are accepted
    nm.tune_import(f"# muon-tune {nm.kernel_hash()}\n# a comment\nnew 0\n")
    nm.tune_import("plain 1\n")
    assert nm.tune_table() == {"keep": 1, "new": 0, "plain": 1}


def test_cache_file_round_trip(clean_table, tmp_path, monkeypatch):
    monkeypatch.setenv("MUON_TUNE_CACHE", str(tmp_path / "tune.txt"))
    assert nm.tune_cache_path() == tmp_path / "tune.txt"
    assert not nm.tune_cache_load()  # no file yet
    nm.tune_import("bf16|0:1:0:640x640*1 1\nf32|2:1:0:64x64*3 0\n")
    path = nm.tune_cache_save()
    assert path.read_text() == nm.tune_export()
    nm.tune_clear()
    assert nm.tune_cache_load()
    assert nm.tune_table() == {"bf16|0:1:0:640x640*1": 1, "f32|2:1:0:64x64*3": 0}


def test_default_cache_path_is_named_for_the_kernels(monkeypatch):
    monkeypatch.delenv("MUON_TUNE_CACHE", raising=False)
    assert nm.tune_cache_path().name == f"tune-{nm.kernel_hash()}.txt"


LIST = [(1024, 4096)] * 3 + [(2048, 2048)]


def _fake_tuner(calls, cfg=1):
    """Stands in for muon_tune (which needs a GPU): records the call and enters a choice for
    every launch of the step, as the tuner does."""
    def run():
        calls.append(1)
        sigs = nm.launch_signatures(nm.shape_array(LIST), len(LIST), nm.make_hparams())
        nm.tune_import("".join(f"{s} {cfg}\n" for s in dict.fromkeys(sigs)))
    return run


def test_a_saved_table_is_reused_without_timing(clean_table, tmp_path):
    arr, hp, cache = nm.shape_array(LIST), nm.make_hparams(), tmp_path / "tune.txt"
    calls = []
    assert nm.tune_with_cache(arr, len(LIST), hp, _fake_tuner(calls), cache) is True
    assert calls == [1] and cache.is_file()
    table = nm.tune_table()
    # a new process: the table is empty; the saved one covers the step, so nothing is timed
    nm.tune_clear()
    assert nm.tune_with_cache(arr, len(LIST), hp, _fake_tuner(calls), cache) is False
    assert calls == [1]
    assert nm.tune_table() == table
    cfgs = [L["cfg"] for L in nm.plan_describe(arr, len(LIST), hp)["launches"] if L["kind"] == "gemm"]
    assert cfgs and all(c == 1 for c in cfgs)


def test_a_stale_or_partial_table_is_timed_again(clean_table, tmp_path):
    arr, hp, cache = nm.shape_array(LIST), nm.make_hparams(), tmp_path / "tune.txt"
    other = "0" * 16 if nm.kernel_hash() != "0" * 16 else "1" * 16
    sigs = nm.launch_signatures(arr, len(LIST), hp)
    cache.write_text(f"# muon-tune {other}\n" + "".join(f"{s} 3\n" for s in dict.fromkeys(sigs)))
    calls = []
    assert nm.tune_with_cache(arr, len(LIST), hp, _fake_tuner(calls), cache) is True
    assert calls == [1]
    assert cache.read_text().splitlines()[0] == f"# muon-tune {nm.kernel_hash()}"
    assert set(nm.tune_table().values()) == {1}
    # a table that covers only part of the step is completed by timing
    nm.tune_clear()
    cache.write_text(f"# muon-tune {nm.kernel_hash()}\n{sigs[0]} 0\n")
    assert nm.tune_with_cache(arr, len(LIST), hp, _fake_tuner(calls), cache) is True
    assert calls == [1, 1]


def test_no_cache_always_times(clean_table):
    arr, hp = nm.shape_array(LIST), nm.make_hparams()
    calls = []
    nm.tune_with_cache(arr, len(LIST), hp, _fake_tuner(calls), cache=False)
    assert calls == [1]
    nm.tune_with_cache(arr, len(LIST), hp, _fake_tuner(calls), cache=False)  # covered already
    assert calls == [1]


def test_a_saved_table_serves_another_process(clean_table, tmp_path):
    """The cache outlives the process: a second interpreter loads it and finds every launch
    of the same step chosen, so it would time nothing."""
    import subprocess
    import sys

    arr, hp, cache = nm.shape_array(LIST), nm.make_hparams(), tmp_path / "tune.txt"
    nm.tune_with_cache(arr, len(LIST), hp, _fake_tuner([], cfg=3), cache)
    code = (
        "import newton_schulz_02_amd as nm\n"
        f"LIST = {LIST!r}\n"
        "arr, hp = nm.shape_array(LIST), nm.make_hparams()\n"
        "def never():\n"
        "    raise SystemExit('timed again')\n"
        f"assert nm.tune_with_cache(arr, len(LIST), hp, never, {str(cache)!r}) is False\n"
        "print(sorted(set(nm.tune_table().values())))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                         cwd=str(Path(__file__).resolve().parents[1]))
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "[3]"
