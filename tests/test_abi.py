"""CPU tests of the C ABI: exported symbols, host-side validation and planning.

No test here launches a kernel.  Calls that pass validation are only made when no GPU
is visible (they then stop at the first HIP call with MUON_EHIP); pointers in these
tests are fake host-side numbers and must never reach a device.
"""

from __future__ import annotations

import ctypes
import math
import re
from pathlib import Path

import pytest

import newton_schulz_02_amd as nm

HEADERS = sorted((Path(__file__).resolve().parents[1] / "include").glob("*.h"))


def _gpu_visible() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


def declared_functions():
    names = []
    for header in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", header.read_text(), flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*([a-z_]+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n.startswith(("muon_", "adamw_", "shampoo_"))))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"muon_step", "muon_workspace_size", "adamw_step", "muon_strerror",
            "muon_last_error", "muon_profile_begin", "muon_profile_end", "shampoo_step",
            "shampoo_workspace_size", "shampoo_plan_describe"} <= set(names)
    lib = nm.lib()
    for name in names:
        assert hasattr(lib, name), name
    assert nm.version().startswith("muon-gfx950")


def test_strerror_covers_every_status():
    for code in (0, -1, -2, -3, -4, -5):
        assert nm.strerror(code) != "unknown status"
    assert nm.strerror(7) == "unknown status"


HP = nm.make_hparams()


def call_step(arr, count, hp=HP, ws=1 << 32, ws_bytes=1 << 40):
    return nm.lib().muon_step(arr, count, ctypes.byref(hp) if hp is not None else None,
                              ctypes.c_void_p(ws), ws_bytes, None)


def mats(*shapes, dtype=nm.MUON_BF16):
    return nm.shape_array([tuple(s) for s in shapes], dtype)


@pytest.mark.parametrize("mutate,code", [
    (lambda a, h: a.__setitem__(0, nm.muon_matrix(0, a[0].grad, a[0].momentum, 8, 8, 1, 0)), nm.MUON_EINVAL),
    (lambda a, h: setattr(a[0], "rows", 0), nm.MUON_EINVAL),
    (lambda a, h: setattr(a[0], "cols", -3), nm.MUON_EINVAL),
    (lambda a, h: setattr(a[0], "cols", (1 << 20) + 1), nm.MUON_EINVAL),
    (lambda a, h: setattr(a[0], "dtype", 7), nm.MUON_EINVAL),
    (lambda a, h: setattr(a[0], "reserved", 1), nm.MUON_EINVAL),
    (lambda a, h: setattr(a[0], "param", a[0].param + 1), nm.MUON_EINVAL),
    (lambda a, h: setattr(h, "lr", float("nan")), nm.MUON_EINVAL),
    (lambda a, h: setattr(h, "beta", float("inf")), nm.MUON_EINVAL),
    (lambda a, h: setattr(h, "eps", -1.0), nm.MUON_EINVAL),
    (lambda a, h: setattr(h, "ns_steps", 32), nm.MUON_EINVAL),
    (lambda a, h: setattr(h, "ns_steps", -1), nm.MUON_EINVAL),
    (lambda a, h: setattr(a[0], "grad", a[0].param), nm.MUON_EALIAS),
    (lambda a, h: setattr(a[0], "momentum", a[0].param), nm.MUON_EALIAS),
    (lambda a, h: setattr(a[1], "param", a[0].momentum + 64), nm.MUON_EALIAS),
    (lambda a, h: setattr(a[1], "grad", a[0].param + 64), nm.MUON_EALIAS),
])
def test_validation_rejects_before_any_hip_call(mutate, code):
    arr = mats((8, 8), (8, 8))
    hp = nm.make_hparams()
    mutate(arr, hp)
    for fn in ("step", "size"):
        if fn == "step":
            rc = call_step(arr, 2, hp)
        else:
            out = ctypes.c_size_t(0)
            rc = nm.lib().muon_workspace_size(arr, 2, ctypes.byref(hp), ctypes.byref(out))
        assert rc == code, (fn, rc, nm.last_error())
        assert nm.last_error()


def test_gradients_may_overlap_each_other():
    arr = mats((8, 8), (8, 8))
    arr[1].grad = arr[0].grad  # shared read-only gradient: allowed
    out = ctypes.c_size_t(0)
    assert nm.lib().muon_workspace_size(arr, 2, ctypes.byref(HP), ctypes.byref(out)) == nm.MUON_OK


def test_null_arguments():
    out = ctypes.c_size_t(0)
    assert nm.lib().muon_workspace_size(None, 1, ctypes.byref(HP), ctypes.byref(out)) == nm.MUON_EINVAL
    assert nm.lib().muon_workspace_size(mats((4, 4)), 1, None, ctypes.byref(out)) == nm.MUON_EINVAL
    assert nm.lib().muon_workspace_size(mats((4, 4)), 1, ctypes.byref(HP), None) == nm.MUON_EINVAL
    assert nm.lib().muon_workspace_size(mats((4, 4)), -1, ctypes.byref(HP), ctypes.byref(out)) == nm.MUON_EINVAL
    assert call_step(mats((4, 4)), 1, ws=0) == nm.MUON_EINVAL
    assert call_step(mats((4, 4)), 1, ws=(1 << 32) + 64) == nm.MUON_EINVAL  # not 256-aligned


def test_workspace_too_small_is_enospc():
    arr = mats((100, 300))
    need = nm.workspace_size_raw(arr, 1, HP)
    assert call_step(arr, 1, ws_bytes=need - 1) == nm.MUON_ENOSPC
    assert "needs" in nm.last_error()


def test_count_zero_is_a_no_op():
    assert call_step(mats((4, 4)), 0) == nm.MUON_OK
    assert nm.workspace_size_raw(mats((4, 4)), 0, HP) == 0


@pytest.mark.skipif(_gpu_visible(), reason="valid call with fake pointers: only without a GPU")
def test_valid_call_without_gpu_reports_hip_error():
    assert call_step(mats((64, 64)), 1) == nm.MUON_EHIP
    assert "hipGetDevice" in nm.last_error()
    hp = nm.adamw_hparams(1e-3, 0.9, 0.95, 1e-8, 0.1, 1)
    rc = nm.lib().adamw_step(ctypes.c_void_p(1 << 20), ctypes.c_void_p(2 << 20), ctypes.c_void_p(3 << 20),
                             ctypes.c_void_p(4 << 20), 16, ctypes.byref(hp), None)
    assert rc == nm.MUON_EHIP


def test_adamw_validation():
    lib = nm.lib()
    P = [ctypes.c_void_p(k << 20) for k in (1, 2, 3, 4)]

    def run(n=16, **kw):
        h = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1)
        h.update(kw)
        hp = nm.adamw_hparams(h["lr"], h["beta1"], h["beta2"], h["eps"], h["weight_decay"], h["step"])
        return lib.adamw_step(*P, n, ctypes.byref(hp), None)

    assert run(step=0) == nm.MUON_EINVAL
    assert run(beta1=1.0) == nm.MUON_EINVAL
    assert run(lr=float("nan")) == nm.MUON_EINVAL
    assert run(n=-1) == nm.MUON_EINVAL
    assert run(n=0) == nm.MUON_OK
    hp = nm.adamw_hparams(1e-3, 0.9, 0.95, 1e-8, 0.1, 1)
    assert lib.adamw_step(P[0], P[0], P[2], P[3], 16, ctypes.byref(hp), None) == nm.MUON_EALIAS
    assert lib.adamw_step(ctypes.c_void_p(2), P[1], P[2], P[3], 16, ctypes.byref(hp), None) == nm.MUON_EINVAL


# --- planning ------------------------------------------------------------------------------

def plan(shapes, dtype=nm.MUON_BF16, **hp):
    arr = mats(*shapes, dtype=dtype)
    return nm.plan_describe(arr, len(shapes), nm.make_hparams(**hp))


@pytest.mark.parametrize("shape,steps,want", [
    ((4096, 4096), 5, {2, 3, 4}),
    ((1024, 1024), 5, {2, 3, 4}),
    ((4096, 11008), 5, set()),
    ((11008, 4096), 5, set()),
    ((1024, 1535), 5, {2, 3, 4}),
    ((1535, 1024), 5, {2, 3, 4}),
    ((1024, 1536), 5, set()),
    ((512, 512), 7, {2, 3, 4, 5, 6}),
    ((512, 512), 3, {2}),
    ((512, 512), 2, set()),
    ((512, 512), 0, set()),
])
def test_auto_restart_sets(shape, steps, want):
    p = plan([shape], steps=steps)
    mask = p["matrices"][0]["restarts"]
    assert {k for k in range(32) if mask >> k & 1} == want


def test_explicit_restart_mask_clips_bit0_and_range():
    p = plan([(64, 64)], restart_mask=0b1111111, steps=5)
    assert p["matrices"][0]["restarts"] == 0b11110


def _flops_rect(m, n, k=5):
    # symmetric m x m x k products count m(m+1)k; full products 2 m n k.
    return m * (m + 1) * n + (4 * k - 3) * m * (m + 1) * m + 2 * m * m * n


def test_flop_count_matches_the_counting_rule():
    p = plan([(4096, 11008)])
    assert p["flops"] == _flops_rect(4096, 11008)
    # Square with restarts {2, 3, 4}: 4 SYRKs, 8 Gram products, 3 re-anchors and the apply.
    m = 4096
    want = 4 * m * (m + 1) * m + 8 * m * (m + 1) * m + 4 * 2 * m ** 3
    assert plan([(m, m)])["flops"] == want


def test_layer_flops_and_launch_count():
    from newton_schulz_02_amd.workloads import WORKLOADS

    wl = WORKLOADS["layer4096_bf16"]
    p = plan([(s.rows, s.cols) for s in wl.matrices])
    assert math.isclose(p["flops"], 1.0666e13, rel_tol=1e-3)
    kinds = [L["kind"] for L in p["launches"]]
    assert kinds.count("momentum") == 1 and kinds.count("norm") == 1
    assert kinds.count("gemm") == p["levels"] <= 17


def test_buckets_are_contiguous_and_sorted():
    shapes = [(256, 256), (512, 2048), (256, 256), (2048, 512), (512, 2048), (256, 256)]
    p = plan(shapes)
    order = [(m["restarts"], m["tall"], m["m"], m["n"]) for m in p["matrices"]]
    assert order == sorted(order)
    assert sorted(m["orig"] for m in p["matrices"]) == list(range(len(shapes)))
    for L in p["launches"]:
        for g in L["groups"]:
            assert 0 <= g["first"] < g["last"] <= len(shapes)


def test_mixed_dtypes_get_separate_launches():
    arr = nm.shape_array([(200, 300, nm.MUON_BF16), (64, 128, nm.MUON_F32)])
    p = nm.plan_describe(arr, 2, HP)
    moms = [L for L in p["launches"] if L["kind"] == "momentum"]
    assert sorted(L["dtype"] for L in moms) == [1, 2]
    for L in p["launches"]:
        if L["kind"] == "gemm":
            dt = {p["matrices"][i]["dtype"] for g in L["groups"] for i in range(g["first"], g["last"])}
            assert dt == {L["dtype"]}


@pytest.mark.parametrize("m", [1, 4, 33, 64, 128, 129, 256])
def test_small_bf16_matrices_iterate_in_fp32(m):
    """bf16 matrices with at most 128 Gram rows run their Gram iteration in fp32: they share
    the fp32 contraction launches (a launch's dtype is its operands'), while their momentum
    launch stays bf16; their workspace forms are fp32."""
    arr = nm.shape_array([(m, 4 * m + 100, nm.MUON_BF16), (300, 700, nm.MUON_BF16),
                          (50, 90, nm.MUON_F32)])
    p = nm.plan_describe(arr, 3, HP)
    small = next(x for x in p["matrices"] if x["orig"] == 0)
    assert small["dtype"] == 1 and small["gram_dtype"] == (2 if m <= 128 else 1)
    assert next(x for x in p["matrices"] if x["orig"] == 1)["gram_dtype"] == 1
    assert next(x for x in p["matrices"] if x["orig"] == 2)["gram_dtype"] == 2
    moms = [L for L in p["launches"] if L["kind"] == "momentum"]
    assert sorted(L["dtype"] for L in moms) == [1, 2]
    for L in p["launches"]:
        if L["kind"] == "gemm":
            gd = {p["matrices"][i]["gram_dtype"] for g in L["groups"] for i in range(g["first"], g["last"])}
            assert gd == {L["dtype"]}
    # Gram slots of the small matrix hold fp32: m x round_up(m, 128) x 4 bytes.
    es = 4 if m <= 128 else 2
    mp = -(-m // 128) * 128
    assert small["regions"][0][1] == m * mp * es


def test_workspace_size_independent_of_pointers_and_grows_with_count():
    a1 = nm.shape_array([(300, 700)])
    a2 = nm.shape_array([(300, 700)])
    a2[0].param += 1 << 36
    a2[0].grad += 1 << 36
    a2[0].momentum += 1 << 36
    s1 = nm.workspace_size_raw(a1, 1, HP)
    assert s1 == nm.workspace_size_raw(a2, 1, HP)
    assert nm.workspace_size_raw(nm.shape_array([(300, 700)] * 2), 2, HP) > s1
    assert s1 % 256 == 0


# --- tile orders of the MFMA kernel --------------------------------------------------------

@pytest.mark.parametrize("T", list(range(1, 20)) + [43, 64])
def test_triangle_order_is_a_bijection_onto_the_lower_triangle(T):
    order = nm.tile_order(True, T)
    assert len(order) == T * (T + 1) // 2
    assert sorted(order) == sorted((i, j) for i in range(T) for j in range(i + 1))
    # Banded: the first tiles stay within the first band of 4 tile rows.
    assert all(i < 4 for i, _ in order[:min(10, len(order))])


@pytest.mark.parametrize("TM,TN", [(1, 1), (1, 7), (5, 3), (16, 43), (43, 16), (9, 9)])
def test_full_order_is_a_bijection(TM, TN):
    order = nm.tile_order(False, TM, TN)
    assert sorted(order) == sorted((i, j) for i in range(TM) for j in range(TN))


@pytest.mark.parametrize("total", [1, 5, 8, 9, 136, 256, 952, 1001, 3088])
def test_xcd_remap_is_a_permutation_dealing_chunks_round_robin(total):
    out = nm.xcd_remap(total)
    assert sorted(out) == list(range(total))
    whole = total // 256 * 256
    rest = total - whole
    tail_of = {x: [] for x in range(8)}
    for w in range(total):
        x, i = w % 8, w // 8
        if w < whole:
            # XCD x (workgroups w = x mod 8) gets chunk x of each round of 8 chunks of 32.
            assert out[w] // 32 % 8 == x and out[w] // 256 == i // 32
        else:
            assert out[w] >= whole
            tail_of[(w - whole) % 8].append(out[w])
    # The tail: XCD x gets one contiguous block of ceil or floor(rest / 8) tiles, in order.
    start = whole
    for x in range(8):
        blk = tail_of[x]
        assert blk == list(range(start, start + len(blk)))
        assert len(blk) in (rest // 8, -(-rest // 8))
        start += len(blk)
    assert start == total


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library every entry point raises; nothing falls back to the CPU."""
    import torch

    monkeypatch.setattr(nm, "LIB_PATH", tmp_path / "libmuon.so")
    monkeypatch.setattr(nm, "_lib", None)
    with pytest.raises(nm.MuonLibraryMissing):
        nm.lib()
    w = torch.zeros(8, 16, dtype=torch.bfloat16)
    with pytest.raises(nm.MuonLibraryMissing):
        nm.MuonStep([w], [w.clone()], [w.clone()], lr=0.02, beta=0.95)
    f = torch.zeros(8, 16)
    with pytest.raises(nm.MuonLibraryMissing):
        nm.ShampooStep([f], [f.clone()], [torch.zeros(8, 8)], [torch.zeros(16, 16)], lr=0.1,
                       beta2=0.9, eps=1e-6, root_iters=4)


def test_product_code_never_reaches_the_oracle():
    """The package and the C sources name no oracle module: the oracle only checks results."""
    root = Path(nm.__file__).resolve().parent
    files = list(root.glob("*.py")) + list((root / "csrc").glob("*"))
    for f in files:
        if f.is_file() and f.suffix in (".py", ".cpp", ".h", ".hip"):
            text = f.read_text()
            assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), f
            assert "oracle/" not in text, f


def test_product_header_holds_no_test_hooks_and_the_library_allocates_no_device_memory():
    """muon.h is the product interface: the host-only test hooks live in muon_test_hooks.h.
    No source of the library calls a device allocator (the caller owns every device buffer;
    the tuner's copies go to caller scratch)."""
    root = Path(__file__).resolve().parents[1]
    product = re.sub(r"/\*.*?\*/", "", (root / "include" / "muon.h").read_text(), flags=re.S)
    assert "muon_debug_" not in product
    hooks = (root / "include" / "muon_test_hooks.h").read_text()
    for name in ("muon_debug_tile_order", "muon_debug_xcd_remap", "muon_debug_split", "muon_debug_flat_loads"):
        assert name in hooks
    for src in (root / "newton_schulz_02_amd" / "csrc").glob("*"):
        text = src.read_text()
        for call in ("hipMalloc(", "hipMallocAsync(", "hipExtMallocWithFlags(", "hipMallocManaged(", "hipFree("):
            assert call not in text, f"{src.name} calls {call}"
