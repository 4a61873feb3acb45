"""Python binding of libmuon, the owner-side Gram Newton-Schulz Muon step for gfx950.

Argument marshalling only: every step of the computation runs in the HIP kernels of
``libmuon.so``.  PyTorch supplies device memory and the current stream.  If the library
has not been built, every call raises ``MuonLibraryMissing``; there is no fallback.

Entry points mirror ``include/muon.h``: :func:`workspace_size`, :func:`muon_step`,
:func:`adamw_step`, :func:`step_cost`, :func:`plan_describe`, :func:`profile_begin`,
:func:`profile_end`, :func:`strerror`, :func:`last_error`, :func:`version`,
:func:`shutdown`; and ``include/shampoo.h``: :func:`shampoo_workspace_size`,
:func:`shampoo_step` (:class:`ShampooStep`), :func:`shampoo_plan_describe`.
"""

from __future__ import annotations

import ctypes
import json
from ctypes import POINTER, c_char, c_char_p, c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_uint32, c_void_p
from pathlib import Path

LIB_PATH = Path(__file__).resolve().with_name("libmuon.so")

MUON_OK = 0
MUON_EINVAL = -1
MUON_ENOSPC = -2
MUON_EALIAS = -3
MUON_EHIP = -4
MUON_EUNSUPPORTED = -5
MUON_ESTALE = -6
MUON_BF16 = 1
MUON_F32 = 2
RESTART_AUTO = 0xFFFFFFFF

#: Coefficients published with Muon (Jordan et al., 2024).  The pages print none.
QUINTIC = (3.4445, -4.7750, 2.0315)


class MuonLibraryMissing(RuntimeError):
    pass


class MuonError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{strerror(status)} ({status}): {detail}")
        self.status = status
        self.detail = detail


class muon_matrix(ctypes.Structure):
    _fields_ = [("param", c_void_p), ("grad", c_void_p), ("momentum", c_void_p),
                ("rows", c_int64), ("cols", c_int64), ("dtype", c_int32), ("reserved", c_int32)]


class muon_hparams(ctypes.Structure):
    _fields_ = [("lr", c_float), ("beta", c_float), ("ns_a", c_float), ("ns_b", c_float),
                ("ns_c", c_float), ("ns_steps", c_int32), ("eps", c_float),
                ("restart_mask", c_uint32)]


class adamw_hparams(ctypes.Structure):
    _fields_ = [("lr", c_float), ("beta1", c_float), ("beta2", c_float), ("eps", c_float),
                ("weight_decay", c_float), ("step", c_int32)]


class muon_kernel_stat(ctypes.Structure):
    _fields_ = [("name", c_char * 32), ("launches", c_int64), ("ms", c_double),
                ("flops", c_double), ("bytes", c_double)]


class shampoo_matrix(ctypes.Structure):
    _fields_ = [("param", c_void_p), ("grad", c_void_p), ("stat_left", c_void_p),
                ("stat_right", c_void_p), ("rows", c_int64), ("cols", c_int64), ("dtype", c_int32),
                ("reserved", c_int32)]


class shampoo_hparams(ctypes.Structure):
    _fields_ = [("lr", c_float), ("beta2", c_float), ("eps", c_float), ("root_iters", c_int32)]


_MATP = POINTER(muon_matrix)
_HPP = POINTER(muon_hparams)
_SMATP = POINTER(shampoo_matrix)
_SHPP = POINTER(shampoo_hparams)
_SIGNATURES = {
    "muon_workspace_size": (c_int, [_MATP, c_int32, _HPP, POINTER(c_size_t)]),
    "muon_step": (c_int, [_MATP, c_int32, _HPP, c_void_p, c_size_t, c_void_p]),
    "adamw_step": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int64, POINTER(adamw_hparams), c_void_p]),
    "muon_step_cost": (c_int, [_MATP, c_int32, _HPP, POINTER(c_double), POINTER(c_double)]),
    "muon_plan_describe": (c_int, [_MATP, c_int32, _HPP, c_char_p, c_size_t]),
    "muon_profile_begin": (c_int, []),
    "muon_profile_end": (c_int, [POINTER(muon_kernel_stat), c_int32, POINTER(c_int32)]),
    "muon_strerror": (c_char_p, [c_int]),
    "muon_last_error": (c_char_p, []),
    "muon_version": (c_char_p, []),
    "muon_shutdown": (None, []),
    "muon_debug_tile_order": (c_int, [c_int, c_int, c_int, POINTER(c_int), POINTER(c_int)]),
    "muon_debug_xcd_remap": (c_int, [c_int, POINTER(c_int)]),
    "muon_owner_assign": (c_int, [POINTER(c_double), c_int32, c_int32, c_int64, POINTER(c_int32),
                                  POINTER(c_double), POINTER(c_int32)]),
    "muon_tune_scratch_size": (c_int, [_MATP, c_int32, _HPP, POINTER(c_size_t)]),
    "muon_tune": (c_int, [_MATP, c_int32, _HPP, c_void_p, c_size_t, c_void_p, c_size_t, c_void_p, c_int32]),
    "muon_tune_force": (c_int, [c_int32]),
    "muon_tune_clear": (None, []),
    "muon_tune_export": (c_int, [c_char_p, c_size_t, POINTER(c_size_t)]),
    "muon_kernel_hash": (c_char_p, []),
    "muon_tune_import": (c_int, [c_char_p]),
    "muon_debug_wide_tile_order": (c_int, [c_int, c_int, c_int, POINTER(c_int), POINTER(c_int)]),
    "muon_debug_split": (c_int, [c_int, c_int, c_int, POINTER(c_int), POINTER(c_int), c_int]),
    "muon_debug_flat_loads": (c_int, [c_int32]),
    "muon_debug_split_spins": (c_int, [c_int32]),
    "muon_debug_split_protocol": (c_int, [c_int32, c_int32, c_int32, POINTER(c_int32)]),
    "muon_workspace_check": (c_int, [c_void_p, c_size_t, c_void_p]),
    "muon_step_noalloc": (c_int, [_MATP, c_int32, _HPP, c_void_p]),
    "shampoo_workspace_size": (c_int, [_SMATP, c_int32, _SHPP, POINTER(c_size_t)]),
    "shampoo_step": (c_int, [_SMATP, c_int32, _SHPP, c_void_p, c_size_t, c_void_p]),
    "shampoo_plan_describe": (c_int, [_SMATP, c_int32, _SHPP, c_char_p, c_size_t]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmuon.so (once).  Raises MuonLibraryMissing if it has not been built."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise MuonLibraryMissing(
                f"{LIB_PATH} not found: build it with `python -m newton_schulz_02_amd.build`")
        # One HIP runtime per process: PyTorch ships its own libamdhip64, and the library's
        # dependency must resolve to that one, not to a second copy loaded ahead of it
        # (device memory and streams come from PyTorch).  So PyTorch loads first.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        handle = ctypes.CDLL(str(LIB_PATH))
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def strerror(status: int) -> str:
    return lib().muon_strerror(int(status)).decode()


def last_error() -> str:
    return lib().muon_last_error().decode()


def version() -> str:
    return lib().muon_version().decode()


def shutdown() -> None:
    lib().muon_shutdown()


def _check(status: int) -> None:
    if status != MUON_OK:
        raise MuonError(status, last_error())


# --- descriptors ------------------------------------------------------------------------

def make_hparams(lr=0.02, beta=0.95, coeffs=QUINTIC, steps=5, eps=1e-7,
                 restart_mask=RESTART_AUTO) -> muon_hparams:
    a, b, c = coeffs
    return muon_hparams(float(lr), float(beta), float(a), float(b), float(c), int(steps),
                        float(eps), int(restart_mask) & 0xFFFFFFFF)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return MUON_BF16
    if t.dtype == torch.float32:
        return MUON_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def matrix_array(params, grads, moms):
    """Pack lists of 2D device tensors into a ctypes muon_matrix array."""
    if not (len(params) == len(grads) == len(moms)):
        raise ValueError("params, grads and moms must have the same length")
    arr = (muon_matrix * max(1, len(params)))()
    for i, (w, g, m) in enumerate(zip(params, grads, moms)):
        for t in (w, g, m):
            if t.dim() != 2 or not t.is_contiguous():
                raise ValueError(f"matrix {i}: tensors must be 2D and contiguous")
            if tuple(t.shape) != tuple(w.shape) or t.dtype != w.dtype:
                raise ValueError(f"matrix {i}: param, grad and momentum must match in shape and dtype")
        arr[i] = muon_matrix(w.data_ptr(), g.data_ptr(), m.data_ptr(), w.shape[0], w.shape[1],
                             _dtype_code(w), 0)
    return arr


def shape_array(shapes, dtype=MUON_BF16):
    """A muon_matrix array with fake, distinct, aligned pointers: for host-only planning calls."""
    arr = (muon_matrix * max(1, len(shapes)))()
    base = 1 << 40
    for i, sh in enumerate(shapes):
        r, c = sh[0], sh[1]
        dt = sh[2] if len(sh) > 2 else dtype
        es = 2 if dt == MUON_BF16 else 4
        nbytes = ((r * c * es + 4095) // 4096) * 4096
        arr[i] = muon_matrix(base, base + nbytes, base + 2 * nbytes, r, c, dt, 0)
        base += 3 * nbytes
    return arr


def _stream_handle(stream, device):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


# --- entry points -----------------------------------------------------------------------

def workspace_size_raw(arr, count: int, hp: muon_hparams) -> int:
    out = c_size_t(0)
    _check(lib().muon_workspace_size(arr, int(count), ctypes.byref(hp), ctypes.byref(out)))
    return int(out.value)


def step_raw(arr, count: int, hp: muon_hparams, ws_ptr: int, ws_bytes: int, stream_ptr) -> None:
    _check(lib().muon_step(arr, int(count), ctypes.byref(hp), c_void_p(ws_ptr), int(ws_bytes),
                           stream_ptr))


def tune_scratch_size_raw(arr, count: int, hp: muon_hparams) -> int:
    n = c_size_t(0)
    _check(lib().muon_tune_scratch_size(arr, int(count), ctypes.byref(hp), ctypes.byref(n)))
    return int(n.value)


def tune_raw(arr, count: int, hp: muon_hparams, ws_ptr: int, ws_bytes: int, scratch_ptr: int,
             scratch_bytes: int, stream_ptr, reps: int = 5) -> None:
    _check(lib().muon_tune(arr, int(count), ctypes.byref(hp), c_void_p(ws_ptr), int(ws_bytes),
                           c_void_p(scratch_ptr), int(scratch_bytes), stream_ptr, int(reps)))


# MFMA kernel configurations: 256 x 256 and 256 x 384 tiles, each also with the tail split,
# the 256 x 256 kernel with the deeper load pipeline (4 LDS stages of 64-byte rows), and
# 128 x 128 tiles (4 waves, three workgroups per compute unit).
CFG_SQUARE, CFG_WIDE, CFG_SQUARE_SPLIT, CFG_WIDE_SPLIT, CFG_SQUARE_DEEP, CFG_SMALL = 0, 1, 2, 3, 4, 5
CFG_LABELS = {0: "256x256", 1: "256x384", 2: "256x256+split", 3: "256x384+split", 4: "256x256 deep",
              5: "128x128"}


def tune_force(cfg) -> None:
    """Force one kernel configuration for every launch (None: use the tuning table)."""
    _check(lib().muon_tune_force(-1 if cfg is None else int(cfg)))


def tune_clear() -> None:
    lib().muon_tune_clear()


def tune_export() -> str:
    """The tuning table as text: one "signature cfg" line per entry."""
    need = c_size_t(0)
    _check(lib().muon_tune_export(None, 0, ctypes.byref(need)))
    buf = ctypes.create_string_buffer(need.value)
    _check(lib().muon_tune_export(buf, need.value, ctypes.byref(need)))
    return buf.value.decode()


def tune_import(text: str) -> None:
    _check(lib().muon_tune_import(text.encode()))


def tune_table() -> dict:
    return {sig: int(c) for sig, c in (ln.rsplit(" ", 1) for ln in tune_export().splitlines()
                                        if ln and not ln.startswith("#"))}


def kernel_hash() -> str:
    """Hash of the kernel sources the library was built from: the version of its tuning tables."""
    return lib().muon_kernel_hash().decode()


def tune_cache_path() -> Path:
    """Where tuning tables persist across processes: $MUON_TUNE_CACHE, else a file named for
    this build's kernels under ~/.cache/newton_schulz_02_amd (so builds never share one)."""
    import os

    env = os.environ.get("MUON_TUNE_CACHE")
    if env:
        return Path(env)
    return Path.home() / ".cache" / "newton_schulz_02_amd" / f"tune-{kernel_hash()}.txt"


def tune_cache_load(path=None) -> bool:
    """Add a saved tuning table to the library's table.  False (and nothing added) when there
    is no such file or it was measured on other kernels."""
    path = Path(path) if path is not None else tune_cache_path()
    if not path.is_file():
        return False
    status = lib().muon_tune_import(path.read_text().encode())
    if status == MUON_ESTALE:
        return False
    _check(status)
    return True


def tune_cache_save(path=None) -> Path:
    """Write the library's table (with its kernel hash) to the cache file, atomically."""
    import os

    path = Path(path) if path is not None else tune_cache_path()
    path.parent.mkdir(parents=True, exist_ok=True)
    tmp = path.with_name(path.name + f".{os.getpid()}.tmp")
    tmp.write_text(tune_export())
    os.replace(tmp, path)
    return path


def launch_signatures(arr, count: int, hp: muon_hparams) -> list:
    """Tuning keys (signatures) of a step's MFMA launches."""
    return [L["signature"] for L in plan_describe(arr, count, hp)["launches"] if L["kind"] == "gemm"]


def tune_with_cache(arr, count: int, hp: muon_hparams, run_tuning, cache=True) -> bool:
    """Pick the kernel configuration of each MFMA launch of a step, reusing saved choices.

    With a cache (True: tune_cache_path(); or a path), a saved table is loaded first; if it
    (with what the process already holds) covers every launch of the step, nothing is timed.
    Otherwise run_tuning() times the step and the merged table is saved.  Returns whether it
    timed anything."""
    path = None if cache is False or cache is None else (tune_cache_path() if cache is True else Path(cache))
    if path is not None:
        tune_cache_load(path)
    table = tune_table()
    if all(sig in table for sig in launch_signatures(arr, count, hp)):
        return False
    run_tuning()
    if path is not None:
        tune_cache_save(path)
    return True


def workspace_size(params, grads, moms, **hp) -> int:
    return workspace_size_raw(matrix_array(params, grads, moms), len(params), make_hparams(**hp))


def step_cost(arr, count: int, hp: muon_hparams) -> tuple[float, float]:
    f, b = c_double(0), c_double(0)
    _check(lib().muon_step_cost(arr, int(count), ctypes.byref(hp), ctypes.byref(f), ctypes.byref(b)))
    return f.value, b.value


def owner_assign(costs, ranks: int, node_limit: int = 1_000_000):
    """Owners for matrices of the given costs (``muon_owner_assign``).

    Returns (owner list, makespan, optimal); optimal is True when the library proved the
    makespan minimal."""
    n = len(costs)
    arr = (c_double * max(n, 1))(*[float(c) for c in costs])
    out = (c_int32 * max(n, 1))()
    mk, opt = c_double(0.0), c_int32(0)
    _check(lib().muon_owner_assign(arr, n, int(ranks), int(node_limit), out, ctypes.byref(mk),
                                   ctypes.byref(opt)))
    return list(out[:n]), mk.value, bool(opt.value)


def plan_describe(arr, count: int, hp: muon_hparams, size: int = 1 << 24) -> dict:
    buf = ctypes.create_string_buffer(size)
    _check(lib().muon_plan_describe(arr, int(count), ctypes.byref(hp), buf, size))
    return json.loads(buf.value.decode())


class MuonStep:
    """A prepared Muon step over fixed lists of device tensors.

    Holds the packed descriptors and a torch-allocated workspace; each call enqueues one
    ``muon_step`` on the current (or given) stream.
    """

    def __init__(self, params, grads, moms, *, lr=0.02, beta=0.95, coeffs=QUINTIC, steps=5,
                 eps=1e-7, restart_mask=RESTART_AUTO, workspace=None):
        import torch

        self.params, self.grads, self.moms = list(params), list(grads), list(moms)
        self.count = len(self.params)
        self.hp = make_hparams(lr, beta, coeffs, steps, eps, restart_mask)
        self.arr = matrix_array(self.params, self.grads, self.moms)
        self.ws_bytes = workspace_size_raw(self.arr, self.count, self.hp)
        self.device = self.params[0].device if self.count else torch.device("cuda")
        if workspace is None:
            workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.device)
        if workspace.numel() < self.ws_bytes:
            raise ValueError(f"workspace has {workspace.numel()} bytes, needs {self.ws_bytes}")
        self.workspace = workspace

    def cost(self) -> tuple[float, float]:
        return step_cost(self.arr, self.count, self.hp)

    def __call__(self, stream=None) -> None:
        step_raw(self.arr, self.count, self.hp, self.workspace.data_ptr(), self.workspace.numel(),
                 _stream_handle(stream, self.device))

    def check(self, stream=None) -> None:
        """Raise MuonError if the last step reported a failure (muon_workspace_check)."""
        workspace_check(self.workspace, stream)

    def tune(self, stream=None, reps: int = 5, cache=False) -> bool:
        """Time every MFMA launch of this step under each kernel configuration and keep the
        fastest (``muon_tune``).  It runs on copies of the params and momenta in a scratch
        tensor allocated here, so they are unchanged; the call synchronises the stream.

        cache (True: tune_cache_path(), or a path) reuses and extends a table saved by an
        earlier process for the same kernels: when it covers this step, nothing is timed.
        Returns whether anything was timed."""
        import torch

        def run_tuning():
            need = tune_scratch_size_raw(self.arr, self.count, self.hp)
            if need == 0:
                return
            s = stream if stream is not None else torch.cuda.current_stream(self.device)
            with torch.cuda.stream(s):
                scratch = torch.empty(need, dtype=torch.uint8, device=self.device)
            tune_raw(self.arr, self.count, self.hp, self.workspace.data_ptr(), self.workspace.numel(),
                     scratch.data_ptr(), scratch.numel(), _stream_handle(s, self.device), reps)

        return tune_with_cache(self.arr, self.count, self.hp, run_tuning, cache)


def muon_step_noalloc(params, grads, moms, *, stream=None, **hp) -> None:
    """One Muon step with no workspace argument and no device allocation (the library's
    per-device scratch array, muon_step_noalloc); calls on one device must not overlap."""
    import torch

    params = list(params)
    if not params:
        return
    dev = params[0].device
    arr = matrix_array(params, list(grads), list(moms))
    h = make_hparams(**hp)
    _check(lib().muon_step_noalloc(arr, len(params), ctypes.byref(h), _stream_handle(stream, dev)))


def noalloc_check(stream=None, device=None) -> None:
    """Raise MuonError if the last muon_step_noalloc on the current device reported a failure."""
    import torch

    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    _check(lib().muon_workspace_check(None, 0, _stream_handle(stream, dev)))


def muon_step(params, grads, moms, *, stream=None, **hp) -> None:
    """One Muon step over lists of device tensors (param and momentum updated in place).

    The throwaway workspace is allocated on the stream the step runs on, so the caching
    allocator does not hand its block to other work before that stream has finished with it.
    """
    import torch

    params = list(params)
    if not params:
        return
    dev = params[0].device
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.stream(s):
        step = MuonStep(params, grads, moms, **hp)
    step(s)


def adamw_step(p, g, m, v, *, lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1,
               step=1, stream=None) -> None:
    """AdamW on packed fp32 device vectors (p, m, v updated in place)."""
    import torch

    for t in (p, g, m, v):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("adamw tensors must be contiguous float32")
        if t.numel() != p.numel():
            raise ValueError("adamw tensors must have the same size")
    hp = adamw_hparams(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), int(step))
    _check(lib().adamw_step(c_void_p(p.data_ptr()), c_void_p(g.data_ptr()), c_void_p(m.data_ptr()),
                            c_void_p(v.data_ptr()), p.numel(), ctypes.byref(hp),
                            _stream_handle(stream, p.device)))


def tile_order(tri: bool, tm: int, tn: int = 0):
    """Test hook: the (ti, tj) order in which the MFMA kernel walks one matrix's tiles."""
    n = tm * (tm + 1) // 2 if tri else tm * tn
    ti, tj = (c_int * max(n, 1))(), (c_int * max(n, 1))()
    lib().muon_debug_tile_order(int(bool(tri)), tm, tn, ti, tj)
    return list(zip(ti[:n], tj[:n]))


def wide_tile_order(tri: bool, rows: int, cols: int = 0):
    """Test hook: the (ti, tj) order of the 256 x 384 configuration over a rows x cols output
    (tri: the tiles meeting the lower triangle of a rows x rows output)."""
    n = lib().muon_debug_wide_tile_order(int(bool(tri)), rows, cols, None, None)
    ti, tj = (c_int * max(n, 1))(), (c_int * max(n, 1))()
    lib().muon_debug_wide_tile_order(int(bool(tri)), rows, cols, ti, tj)
    return list(zip(ti[:n], tj[:n]))


def split_plan(tiles: int, units: int, ksteps: int):
    """Test hook: the tail split of a launch.  Returns (plan dict, items) where items[j] is
    (tile, piece, pieces, k0, k1) of tail workgroup j, or None for a padding workgroup."""
    plan = (c_int * 6)()
    n = lib().muon_debug_split(tiles, units, ksteps, plan, None, 0)
    if n < 0:
        _check(n)
    items = (c_int * max(5 * n, 1))()
    lib().muon_debug_split(tiles, units, ksteps, plan, items, n)
    keys = ("mode", "pieces_or_n", "dp_tiles", "tail", "tail_wgs", "slots")
    out = [None if items[5 * j] < 0 else tuple(items[5 * j:5 * j + 5]) for j in range(n)]
    return dict(zip(keys, plan[:6])), out


def flat_loads(on: bool) -> None:
    """Test hook: 64-bit operand pointers in every 256 x 256 launch (the path of operands of
    2 GB and more) instead of 32-bit buffer offsets."""
    _check(lib().muon_debug_flat_loads(1 if on else 0))


def split_spins(spins) -> None:
    """Polls of a tail-split last piece's bounded wait (None: the default)."""
    _check(lib().muon_debug_split_spins(-1 if spins is None else int(spins)))


def split_protocol(pieces: int, mode: int, spin_limit: int) -> list[int]:
    """Host emulation of the tail split's counter protocol (muon_debug_split_protocol)."""
    out = (c_int32 * 8)()
    _check(lib().muon_debug_split_protocol(int(pieces), int(mode), int(spin_limit), out))
    return list(out)


def workspace_check(workspace, stream=None) -> None:
    """Raise MuonError if the last step on this workspace (a torch uint8 tensor) reported a
    failure through its status word; synchronises the stream and clears the word."""
    _check(lib().muon_workspace_check(c_void_p(workspace.data_ptr()), int(workspace.numel()),
                                      _stream_handle(stream, workspace.device)))


def xcd_remap(total: int):
    """Test hook: logical tile of each workgroup id in a grid of `total`."""
    out = (c_int * max(total, 1))()
    lib().muon_debug_xcd_remap(total, out)
    return list(out[:total])


def profile_begin() -> None:
    _check(lib().muon_profile_begin())


def profile_end() -> dict:
    """Stop per-launch timing and return {kernel: {launches, ms, flops, bytes}}."""
    out = (muon_kernel_stat * 16)()
    n = c_int32(0)
    _check(lib().muon_profile_end(out, 16, ctypes.byref(n)))
    return {out[i].name.decode(): {"launches": out[i].launches, "ms": out[i].ms,
                                   "flops": out[i].flops, "bytes": out[i].bytes}
            for i in range(min(n.value, 16))}


# --- Shampoo (include/shampoo.h) --------------------------------------------------------

def make_shampoo_hparams(lr=0.01, beta2=1.0, eps=1e-6, root_iters=20) -> shampoo_hparams:
    return shampoo_hparams(float(lr), float(beta2), float(eps), int(root_iters))


def shampoo_matrix_array(params, grads, lefts, rights):
    """Pack lists of device tensors into a ctypes shampoo_matrix array: param and grad rows x cols
    (float32, or bfloat16 for both), left statistic rows x rows and right statistic cols x cols
    (float32)."""
    import torch

    if not (len(params) == len(grads) == len(lefts) == len(rights)):
        raise ValueError("params, grads, lefts and rights must have the same length")
    arr = (shampoo_matrix * max(1, len(params)))()
    for i, (w, g, lt, rt) in enumerate(zip(params, grads, lefts, rights)):
        r, c = (w.shape[0], w.shape[1]) if w.dim() == 2 else (0, 0)
        want = {"param": (w, (r, c)), "grad": (g, (r, c)), "left": (lt, (r, r)), "right": (rt, (c, c))}
        for name, (t, shape) in want.items():
            if t.dim() != 2 or not t.is_contiguous() or tuple(t.shape) != shape:
                raise ValueError(f"matrix {i}: {name} must be a contiguous {shape[0]} x {shape[1]} tensor")
        if g.dtype != w.dtype:
            raise TypeError(f"matrix {i}: param and grad must have the same dtype")
        if lt.dtype != torch.float32 or rt.dtype != torch.float32:
            raise TypeError(f"matrix {i}: the statistics must be float32")
        arr[i] = shampoo_matrix(w.data_ptr(), g.data_ptr(), lt.data_ptr(), rt.data_ptr(), r, c,
                                _dtype_code(w), 0)
    return arr


def shampoo_shape_array(shapes, dtype=MUON_F32):
    """A shampoo_matrix array with fake, distinct, aligned pointers: for host-only planning calls.
    A shape may carry a third entry, its dtype."""
    arr = (shampoo_matrix * max(1, len(shapes)))()
    base = 1 << 40
    page = lambda n: ((n * 4 + 4095) // 4096) * 4096  # noqa: E731
    for i, sh in enumerate(shapes):
        r, c = sh[0], sh[1]
        dt = sh[2] if len(sh) > 2 else dtype
        w, g, lt, rt = base, base + page(r * c), base + 2 * page(r * c), base + 2 * page(r * c) + page(r * r)
        arr[i] = shampoo_matrix(w, g, lt, rt, r, c, dt, 0)
        base = rt + page(c * c)
    return arr


def shampoo_workspace_size_raw(arr, count: int, hp: shampoo_hparams) -> int:
    out = c_size_t(0)
    _check(lib().shampoo_workspace_size(arr, int(count), ctypes.byref(hp), ctypes.byref(out)))
    return int(out.value)


def shampoo_step_raw(arr, count: int, hp: shampoo_hparams, ws_ptr: int, ws_bytes: int, stream_ptr) -> None:
    _check(lib().shampoo_step(arr, int(count), ctypes.byref(hp), c_void_p(ws_ptr), int(ws_bytes),
                              stream_ptr))


def shampoo_plan_describe(arr, count: int, hp: shampoo_hparams, size: int = 1 << 24) -> dict:
    buf = ctypes.create_string_buffer(size)
    _check(lib().shampoo_plan_describe(arr, int(count), ctypes.byref(hp), buf, size))
    return json.loads(buf.value.decode())


def shampoo_workspace_size(params, grads, lefts, rights, **hp) -> int:
    return shampoo_workspace_size_raw(shampoo_matrix_array(params, grads, lefts, rights), len(params),
                                      make_shampoo_hparams(**hp))


class ShampooStep:
    """A prepared Shampoo step over fixed lists of fp32 device tensors (params and both
    statistics updated in place by each call)."""

    def __init__(self, params, grads, lefts, rights, *, lr=0.01, beta2=1.0, eps=1e-6, root_iters=20,
                 workspace=None):
        import torch

        self.params, self.grads = list(params), list(grads)
        self.lefts, self.rights = list(lefts), list(rights)
        self.count = len(self.params)
        self.hp = make_shampoo_hparams(lr, beta2, eps, root_iters)
        self.arr = shampoo_matrix_array(self.params, self.grads, self.lefts, self.rights)
        self.ws_bytes = shampoo_workspace_size_raw(self.arr, self.count, self.hp)
        self.device = self.params[0].device if self.count else torch.device("cuda")
        if workspace is None:
            workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.device)
        if workspace.numel() < self.ws_bytes:
            raise ValueError(f"workspace has {workspace.numel()} bytes, needs {self.ws_bytes}")
        self.workspace = workspace

    def check(self, stream=None) -> None:
        """Raise MuonError if the last step reported a failure (muon_workspace_check)."""
        workspace_check(self.workspace, stream)

    def plan(self) -> dict:
        return shampoo_plan_describe(self.arr, self.count, self.hp)

    def __call__(self, stream=None) -> None:
        shampoo_step_raw(self.arr, self.count, self.hp, self.workspace.data_ptr(), self.workspace.numel(),
                         _stream_handle(stream, self.device))


def shampoo_step(params, grads, lefts, rights, *, stream=None, **hp) -> None:
    """One Shampoo step over lists of fp32 device tensors.  As muon_step, the throwaway
    workspace is allocated on the stream the step runs on."""
    import torch

    params = list(params)
    if not params:
        return
    dev = params[0].device
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    with torch.cuda.stream(s):
        step = ShampooStep(params, grads, lefts, rights, **hp)
    step(s)
