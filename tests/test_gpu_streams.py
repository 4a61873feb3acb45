"""Calls on several streams and from several host threads.

The library is reentrant when each call in flight has its own workspace: descriptors are
staged through a pinned ring whose slots are reused only after their copy has left, and all
of a call's work goes to its own stream.  Each case runs the same calls twice, once
interleaved over two streams (default priority) or two host threads and once in order on
one stream, and requires bitwise-equal results (every kernel is deterministic)."""

from __future__ import annotations

import threading

import pytest
import torch

import newton_schulz_02_amd as nm
from newton_schulz_02_amd import workloads as W
from tests.gpu_helpers import DEV, log

pytestmark = pytest.mark.gpu


def _muon_state(shapes, seed):
    wl = W.custom("st", shapes, seed=seed)
    items = list(W.generate(wl, weights="random"))
    return wl, [[t.clone() for t in (w, g, m)] for _, w, g, m in items]


def _muon_step(wl, state):
    dev = [[t.to(DEV) for t in x] for x in state]
    step = nm.MuonStep([x[0] for x in dev], [x[1] for x in dev], [x[2] for x in dev], lr=wl.lr,
                       beta=wl.beta, coeffs=wl.coeffs, steps=wl.steps, eps=wl.eps)
    return step, dev


def _shampoo_step(shapes, seed):
    items = list(W.shampoo_inputs(shapes, seed))
    dev = [[t.to(DEV) for t in x] for x in items]
    step = nm.ShampooStep([x[0] for x in dev], [x[1] for x in dev], [x[2] for x in dev],
                          [x[3] for x in dev], lr=0.05, beta2=0.9, eps=1e-6, root_iters=6)
    return step, dev


def _snapshot(dev):
    return [[t.cpu() for t in x] for x in dev]


def _same(a, b):
    return all(torch.equal(x, y) for xa, ya in zip(a, b) for x, y in zip(xa, ya))


def test_two_muon_lists_on_two_streams():
    log("streams: two muon lists")
    wl1, s1 = _muon_state([(512, 1024), (256, 256)], 1)
    wl2, s2 = _muon_state([(768, 768), (1024, 300)], 2)
    # in order on the current stream
    a, da = _muon_step(wl1, s1)
    b, db = _muon_step(wl2, s2)
    for _ in range(4):
        a()
        b()
    torch.cuda.synchronize()
    ref1, ref2 = _snapshot(da), _snapshot(db)
    # interleaved over two streams
    a, da = _muon_step(wl1, s1)
    b, db = _muon_step(wl2, s2)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(4):
        a(sa)
        b(sb)
    torch.cuda.synchronize()
    assert _same(_snapshot(da), ref1) and _same(_snapshot(db), ref2)


def test_muon_and_shampoo_on_two_streams():
    log("streams: muon and shampoo")
    wl, s = _muon_state([(640, 896)], 3)
    m, dm = _muon_step(wl, s)
    sh, dsh = _shampoo_step([(200, 300), (129, 513)], 4)
    for _ in range(3):
        m()
        sh()
    torch.cuda.synchronize()
    ref_m, ref_s = _snapshot(dm), _snapshot(dsh)
    m, dm = _muon_step(wl, s)
    sh, dsh = _shampoo_step([(200, 300), (129, 513)], 4)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        m(s1)
        sh(s2)
    torch.cuda.synchronize()
    assert _same(_snapshot(dm), ref_m) and _same(_snapshot(dsh), ref_s)


def test_two_host_threads():
    log("streams: two host threads")
    wl1, s1 = _muon_state([(512, 512), (300, 700)], 5)
    wl2, s2 = _muon_state([(1024, 256)], 6)
    a, da = _muon_step(wl1, s1)
    b, db = _muon_step(wl2, s2)
    for _ in range(5):
        a()
    for _ in range(5):
        b()
    torch.cuda.synchronize()
    ref1, ref2 = _snapshot(da), _snapshot(db)
    a, da = _muon_step(wl1, s1)
    b, db = _muon_step(wl2, s2)
    errors = []

    def run(step):
        try:
            torch.cuda.set_device(0)
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(5):
                    step(s)
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    ts = [threading.Thread(target=run, args=(x,)) for x in (a, b)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=120)
    assert not errors, errors
    assert not any(t.is_alive() for t in ts)
    torch.cuda.synchronize()
    assert _same(_snapshot(da), ref1) and _same(_snapshot(db), ref2)
