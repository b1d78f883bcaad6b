"""Host-side tests of libtri (no GPU needed): the library loads and exports every function that
include/tri.h declares, the host fold matches the fp64 oracle, and argument checks return their
status codes before any HIP call (fake device addresses are never dereferenced on the host)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

tri = pytest.importorskip("rotary_frequency_key_amd")
from rotary_frequency_key_amd import _abi  # noqa: E402

lib = _abi._lib
OK, ARG, UNSUP, ALIAS, WS = 0, -1, -2, -3, -4


def test_exports_every_declared_function():
    header = open(os.path.join(ROOT, "include", "tri.h")).read()
    header = re.sub(r"/\*.*?\*/", "", header, flags=re.S)
    declared = set(re.findall(r"\b(tri_[a-z0-9_]+)\s*\(", header))
    assert {"tri_fold_weights", "tri_score", "tri_select_topb", "tri_compact_kv"} <= declared
    for name in declared:
        assert hasattr(lib, name), name
    for st in [0, -1, -2, -3, -4, -5, -99]:
        assert lib.tri_status_string(st)


def test_fold_weights_match_oracle():
    D = O.power_of_two_offsets()
    rng = np.random.default_rng(1)
    for d, theta in [(128, 1e4), (128, 1e6), (128, 5e5), (64, 1e4), (256, 1e6), (8, 3.0)]:
        centers = (rng.standard_normal((5, d)) * 2).astype(np.float32)
        W, mu = tri.tri_fold_weights(d, theta, D, centers)
        Wref = O.fold_weights(O.rotary_frequencies(d, theta), D)
        # omega_f from two fp64 pow implementations may differ by an ulp; at offset 2^16 that
        # moves the phase by <= 2^16 * 2^-52 rad, so W agrees to ~1.5e-11 / 17 per term.
        assert np.max(np.abs(W[:, 0] + 1j * W[:, 1] - Wref)) < 1e-12
        mref = O.folded_center(O.as_bands(centers.astype(np.float64)), Wref)
        got = mu[..., 0].astype(np.float64) + 1j * mu[..., 1].astype(np.float64)
        # one binary32 rounding of each component
        err = np.abs(got - mref)
        bound = (np.abs(mref.real) + np.abs(mref.imag)) * 2.0 ** -24 + 1e-12
        assert np.all(err <= bound * 1.01)
    # arbitrary schedule, including 0 and negative offsets
    W, _ = tri.tri_fold_weights(16, 100.0, [0, -3, 5, 7, 7], None)
    Wref = O.fold_weights(O.rotary_frequencies(16, 100.0), [0, -3, 5, 7, 7])
    assert np.max(np.abs(W[:, 0] + 1j * W[:, 1] - Wref)) < 1e-14


def test_fold_weights_errors():
    W = np.zeros((64, 2))
    D = O.power_of_two_offsets()
    dp = D.ctypes.data_as(ctypes.c_void_p)
    wp = W.ctypes.data_as(ctypes.c_void_p)
    assert lib.tri_fold_weights(127, 1e4, dp, 17, None, 0, wp, None) == ARG
    assert lib.tri_fold_weights(128, -1.0, dp, 17, None, 0, wp, None) == ARG
    assert lib.tri_fold_weights(128, float("nan"), dp, 17, None, 0, wp, None) == ARG
    assert lib.tri_fold_weights(128, 1e4, dp, 0, None, 0, wp, None) == ARG
    assert lib.tri_fold_weights(128, 1e4, None, 17, None, 0, wp, None) == ARG
    assert lib.tri_fold_weights(128, 1e4, dp, 17, None, 0, None, None) == ARG
    assert lib.tri_fold_weights(128, 1e4, dp, 17, None, 0, wp, None) == OK


# fake, never-dereferenced device addresses, 256-byte aligned and far apart
A = {k: 0x10_0000_0000 * (i + 1) for i, k in enumerate(
    ["keys", "row_off", "pos", "t", "mu", "scores", "ws", "kidx", "kcnt", "V", "Ko", "Vo", "po"])}


def _score(**kw):
    args = dict(keys=A["keys"], dtype=1, layout=0, d=128, theta=1e6, row_off=A["row_off"], U=8,
                R=262144, maxr=32768, pos=A["pos"], t=A["t"], mu=A["mu"], scores=A["scores"],
                ws=None, wsb=None)
    args.update(kw)
    return lib.tri_score(args["keys"], args["dtype"], args["layout"], args["d"], args["theta"],
                         args["row_off"], args["U"], args["R"], args["maxr"], args["pos"], args["t"],
                         args["mu"], args["scores"], args["ws"], args["wsb"], None)


def test_score_argument_errors():
    assert _score(dtype=7) == ARG
    assert _score(layout=3) == ARG
    assert _score(d=96) == UNSUP
    assert _score(d=127) == ARG
    assert _score(theta=0.0) == ARG
    assert _score(U=0) == ARG
    assert _score(R=-1) == ARG
    assert _score(maxr=1 << 31) == ARG
    assert _score(keys=A["keys"] + 8) == ARG  # misaligned
    assert _score(mu=A["mu"] + 4) == ARG
    assert _score(layout=0x102) == ARG  # unknown band layout under the rotated-keys flag
    assert _score(layout=0x200) == ARG  # unknown flag
    assert _score(keys=None) == ARG
    assert _score(row_off=None) == ARG
    # scores overlapping the keys / positions
    assert _score(scores=A["keys"] + 4096) == ALIAS
    assert _score(scores=A["pos"] - 16) == ALIAS
    # workspace protocol
    n = ctypes.c_size_t(0)
    assert _score(ws=None, wsb=ctypes.byref(n)) == OK and n.value == 8 * 4096 * 4
    small = ctypes.c_size_t(n.value - 1)
    assert _score(ws=A["ws"], wsb=ctypes.byref(small)) == WS
    full = ctypes.c_size_t(n.value)
    assert _score(ws=A["scores"] + 256, wsb=ctypes.byref(full)) == ALIAS
    assert _score(ws=A["ws"] + 16, wsb=ctypes.byref(full)) == ARG  # 256-byte alignment


def _select(**kw):
    args = dict(scores=A["scores"], row_off=A["row_off"], U=8, R=262144, maxr=32768, B=2048,
                kidx=A["kidx"], kcnt=A["kcnt"], ws=None, wsb=None, flags=0)
    args.update(kw)
    return lib.tri_select_topb(args["scores"], args["row_off"], args["U"], args["R"], args["maxr"],
                               args["B"], args["kidx"], args["kcnt"], args["ws"], args["wsb"],
                               args["flags"], None)


def test_select_argument_errors():
    assert _select(B=-1) == ARG
    assert _select(U=0) == ARG
    assert _select(flags=2) == ARG
    assert _select(kcnt=None) == ARG
    assert _select(kidx=None) == ARG
    assert _select(scores=A["scores"] + 2) == ARG
    assert _select(maxr=(1 << 27) + 1, R=(1 << 27) + 1, U=1) == UNSUP  # beyond the select's unit size
    assert _select(flags=1) == WS  # no workspace
    assert _select(flags=0) == WS
    n = ctypes.c_size_t(1)
    assert _select(flags=1, wsb=ctypes.byref(n)) == OK
    size = n.value
    # histograms, unit states (32 bytes each), candidate counts of 32 workgroups of 1024 rows,
    # one candidate word per row, and three words per granule of 64 rows (512 per unit)
    assert size == 8 * 4096 * 4 + 8 * 32 + 8 * 32 * 4 + 8 * 32768 * 4 + 3 * 8 * 512 * 4
    n2 = ctypes.c_size_t(0)
    assert _select(flags=0, wsb=ctypes.byref(n2)) == OK and n2.value == size
    ok = ctypes.c_size_t(size)
    assert _select(ws=A["ws"], wsb=ctypes.byref(ctypes.c_size_t(size - 1))) == WS
    assert _select(ws=A["ws"] + 128, wsb=ctypes.byref(ok)) == ARG  # 256-byte alignment
    assert _select(ws=A["scores"] + 256, wsb=ctypes.byref(ok)) == ALIAS
    assert _select(kcnt=A["kidx"] + 64, ws=A["ws"], wsb=ctypes.byref(ok)) == ALIAS
    assert _select(kidx=A["scores"] + 64, ws=A["ws"], wsb=ctypes.byref(ok)) == ALIAS


def _prune(**kw):
    n = ctypes.c_size_t(1 << 40)
    args = dict(K=A["keys"], V=A["V"], dtype=1, layout=0, d=128, theta=1e6, row_off=A["row_off"], U=8,
                R=262144, maxr=32768, pos=A["pos"], t=A["t"], mu=A["mu"], B=2048, scores=A["scores"],
                kidx=A["kidx"], kcnt=A["kcnt"], Ko=A["Ko"], Vo=A["Vo"], po=A["po"], ws=A["ws"],
                wsb=ctypes.byref(n))
    args.update(kw)
    return lib.tri_prune_pass(*args.values(), None)


def test_prune_pass_argument_errors():
    n = ctypes.c_size_t(0)
    assert _prune(ws=None, wsb=ctypes.byref(n)) == OK and n.value > 0
    assert _prune(ws=None, wsb=None) == WS
    assert _prune(wsb=ctypes.byref(ctypes.c_size_t(16))) == WS
    assert _prune(dtype=3) == ARG
    assert _prune(d=96) == UNSUP
    assert _prune(B=-1) == ARG
    assert _prune(Ko=A["keys"]) == ALIAS
    assert _prune(Vo=A["scores"]) == ALIAS
    assert _prune(po=A["ws"] + 64) == ALIAS
    assert _prune(scores=A["kidx"]) == ALIAS
    assert _prune(kcnt=A["scores"] + 64) == ALIAS
    assert _prune(V=A["V"] + 8) == ARG


def _prune_max(offsets=(1, 2, 4), **kw):
    offs = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    n = ctypes.c_size_t(1 << 40)
    args = dict(K=A["keys"], V=A["V"], dtype=1, layout=0, d=128, theta=1e6,
                offs=offs.ctypes.data_as(ctypes.c_void_p), noffs=offs.size, row_off=A["row_off"], U=8,
                R=262144, maxr=32768, pos=A["pos"], t=A["t"], centers=A["mu"], B=2048, scores=A["scores"],
                kidx=A["kidx"], kcnt=A["kcnt"], Ko=A["Ko"], Vo=A["Vo"], po=A["po"], ws=A["ws"],
                wsb=ctypes.byref(n))
    args.update(kw)
    return lib.tri_prune_pass_max(*args.values(), None)


def test_prune_pass_max_argument_errors():
    n, m = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert _prune_max(ws=None, wsb=ctypes.byref(n)) == OK
    assert _prune(ws=None, wsb=ctypes.byref(m)) == OK and n.value == m.value  # tri_prune_pass's workspace
    assert _prune_max(ws=None, wsb=None) == WS
    assert _prune_max(wsb=ctypes.byref(ctypes.c_size_t(16))) == WS
    assert _prune_max(offsets=[]) == ARG
    assert _prune_max(offs=None) == ARG
    assert _prune_max(offsets=[1, -1]) == ARG
    assert _prune_max(offsets=[1 << 24]) == ARG
    assert _prune_max(offsets=list(range(33))) == UNSUP
    assert _prune_max(layout=0x100, pos=None, po=None, d=96) == UNSUP  # rotated keys: no positions needed
    assert _prune_max(layout=0x100, pos=None, po=None, Ko=A["keys"]) == ALIAS
    assert _prune_max(dtype=3) == ARG
    assert _prune_max(d=96) == UNSUP
    assert _prune_max(B=-1) == ARG
    assert _prune_max(pos=None) == ARG
    assert _prune_max(Ko=A["keys"]) == ALIAS
    assert _prune_max(scores=A["kidx"]) == ALIAS
    assert _prune_max(V=A["V"] + 8) == ARG


def _compact(**kw):
    args = dict(K=A["keys"], V=A["V"], pos=A["pos"], dtype=1, d=128, row_off=A["row_off"], U=8,
                R=262144, kidx=A["kidx"], kcnt=A["kcnt"], B=2048, Ko=A["Ko"], Vo=A["Vo"], po=A["po"])
    args.update(kw)
    return lib.tri_compact_kv(args["K"], args["V"], args["pos"], args["dtype"], args["d"],
                              args["row_off"], args["U"], args["R"], args["kidx"], args["kcnt"],
                              args["B"], args["Ko"], args["Vo"], args["po"], None)


def test_compact_argument_errors():
    assert _compact(d=96) == UNSUP  # 192-byte rows
    assert _compact(dtype=5) == ARG
    assert _compact(B=-2) == ARG
    assert _compact(pos=None) == ARG  # pos_out without pos
    assert _compact(Ko=A["Ko"] + 4) == ARG
    assert _compact(Ko=A["keys"] + 256) == ALIAS
    assert _compact(Vo=A["Ko"] + 256) == ALIAS
    assert _compact(po=A["kidx"]) == ALIAS
    assert _compact(Ko=A["V"] + 1024) == ALIAS


def _inplace(**kw):
    args = dict(K=A["keys"], V=A["V"], pos=A["pos"], dtype=1, layout=0, d=128, theta=1e6, row_off=A["row_off"],
                U=8, R=8 * 13024, maxr=13024, t=A["t"], mu=A["mu"], B=12000, scores=A["scores"], kcnt=A["kcnt"],
                ws=None, wsb=None)
    args.update(kw)
    return lib.tri_prune_inplace(args["K"], args["V"], args["pos"], args["dtype"], args["layout"], args["d"],
                                 args["theta"], args["row_off"], args["U"], args["R"], args["maxr"], args["t"],
                                 args["mu"], args["B"], args["scores"], args["kcnt"], args["ws"], args["wsb"], None)


def test_prune_inplace_argument_errors():
    n = ctypes.c_size_t(0)
    assert _inplace(wsb=ctypes.byref(n)) == OK
    # the select workspace of 8 x 13024 rows, then two lists of min(B, max_rows - B) = 1024 words per unit
    m = ctypes.c_size_t(0)
    assert _select(maxr=13024, wsb=ctypes.byref(m)) == OK
    assert n.value == m.value + 2 * 8 * 1024 * 4
    ok = ctypes.byref(ctypes.c_size_t(n.value))
    assert _inplace(B=-1, ws=A["ws"], wsb=ok) == ARG
    assert _inplace(kcnt=None, ws=A["ws"], wsb=ok) == ARG
    assert _inplace(V=None, ws=A["ws"], wsb=ok) == ARG
    assert _inplace(pos=None, ws=A["ws"], wsb=ok) == ARG  # positions are read unless the keys are rotated
    assert _inplace(V=A["keys"] + 4096, ws=A["ws"], wsb=ok) == ALIAS  # V overlaps K
    assert _inplace(kcnt=A["pos"] + 64, ws=A["ws"], wsb=ok) == ALIAS
    assert _inplace(ws=A["ws"], wsb=ctypes.byref(ctypes.c_size_t(n.value - 1))) == WS
    assert _inplace(ws=None, wsb=None) == WS
    assert _inplace(maxr=(1 << 27) + 1, R=(1 << 27) + 1, U=1, ws=A["ws"], wsb=ok) == UNSUP


def _score_max(offsets=(1, 2, 4), **kw):
    offs = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    args = dict(keys=A["keys"], dtype=1, layout=0, d=128, theta=1e6, row_off=A["row_off"], U=8,
                R=262144, maxr=32768, pos=A["pos"], t=A["t"], mu=A["mu"], scores=A["scores"],
                ws=None, wsb=None, n=offs.size)
    args.update(kw)
    return lib.tri_score_max(args["keys"], args["dtype"], args["layout"], args["d"], args["theta"],
                             offs.ctypes.data_as(ctypes.c_void_p), args["n"], args["row_off"], args["U"],
                             args["R"], args["maxr"], args["pos"], args["t"], args["mu"], args["scores"],
                             args["ws"], args["wsb"], None)


def test_score_max_argument_errors():
    n = ctypes.c_size_t(0)
    assert _score_max(ws=None, wsb=ctypes.byref(n)) == OK and n.value == 8 * 4096 * 4
    assert _score_max(offsets=[]) == ARG
    assert _score_max(offsets=[1, -1]) == ARG
    assert _score_max(offsets=[1 << 24]) == ARG
    assert _score_max(offsets=list(range(33))) == UNSUP
    # rotated keys need no positions: the call gets past that check to the next one
    assert _score_max(layout=0x100, pos=None, d=96) == UNSUP
    assert _score_max(layout=0x100, pos=None, scores=A["keys"] + 4096) == ALIAS
    assert _score_max(pos=None) == ARG
    assert _score_max(d=96) == UNSUP
    assert _score_max(scores=A["keys"] + 4096) == ALIAS
