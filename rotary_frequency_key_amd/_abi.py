"""ctypes binding of libtri.so. Argument marshalling only: shapes, dtypes and devices of torch
tensors are checked, pointers and the current stream are passed through, and a negative status
from the library raises ``TriError``. No arithmetic of the pass happens here."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

TRI_OK = 0
TRI_DT_F32 = 0
TRI_DT_BF16 = 1
TRI_BANDS_INTERLEAVED = 0
TRI_BANDS_HALF_SPLIT = 1
TRI_KEYS_ROTATED = 0x100  # OR into a layout: keys stored after the rotary rotation
TRI_SELECT_HIST_FROM_SCORE = 1
NOALLOC_SCRATCH_BYTES = 64 << 20  # TRI_NOALLOC_SCRATCH_BYTES: tri_prune_pass_noalloc's static workspace

_HERE = os.path.dirname(os.path.abspath(__file__))
# TRI_LIBRARY names another build of the same library (the host-sanitizer build of the CPU tests,
# or libtri_stamps.so, the measurement build with per-workgroup timestamps)
_LIB_PATH = os.environ.get("TRI_LIBRARY") or os.path.join(_HERE, "libtri.so")


def library_path() -> str:
    return _LIB_PATH


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is not built: run `python -m rotary_frequency_key_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint
    szp = ctypes.POINTER(ctypes.c_size_t)
    lib.tri_status_string.argtypes = [i32]
    lib.tri_status_string.restype = ctypes.c_char_p
    lib.tri_fold_weights.argtypes = [i32, ctypes.c_double, vp, i32, vp, i32, vp, vp]
    lib.tri_fold_weights.restype = i32
    lib.tri_score.argtypes = [vp, i32, i32, i32, ctypes.c_double, vp, i32, i64, i64, vp, vp, vp,
                              vp, vp, szp, vp]
    lib.tri_score.restype = i32
    lib.tri_select_topb.argtypes = [vp, vp, i32, i64, i64, i32, vp, vp, vp, szp, u32, vp]
    lib.tri_select_topb.restype = i32
    lib.tri_compact_kv.argtypes = [vp, vp, vp, i32, i32, vp, i32, i64, vp, vp, i32, vp, vp, vp, vp]
    lib.tri_compact_kv.restype = i32
    lib.tri_prune_pass.argtypes = [vp, vp, i32, i32, i32, ctypes.c_double, vp, i32, i64, i64, vp, vp, vp, i32,
                                   vp, vp, vp, vp, vp, vp, vp, szp, vp]
    lib.tri_prune_pass.restype = i32
    lib.tri_prune_pass_noalloc.argtypes = [vp, vp, i32, i32, i32, ctypes.c_double, vp, i32, i64, i64, vp, vp, vp,
                                           i32, vp, vp, vp, vp, vp, vp, vp]
    lib.tri_prune_pass_noalloc.restype = i32
    lib.tri_score_max.argtypes = [vp, i32, i32, i32, ctypes.c_double, vp, i32, vp, i32, i64, i64, vp, vp, vp,
                                  vp, vp, szp, vp]
    lib.tri_score_max.restype = i32
    lib.tri_prune_pass_max.argtypes = [vp, vp, i32, i32, i32, ctypes.c_double, vp, i32, vp, i32, i64, i64, vp, vp,
                                       vp, i32, vp, vp, vp, vp, vp, vp, vp, szp, vp]
    lib.tri_prune_pass_max.restype = i32
    lib.tri_prune_inplace.argtypes = [vp, vp, vp, i32, i32, i32, ctypes.c_double, vp, i32, i64, i64, vp, vp, i32,
                                      vp, vp, vp, szp, vp]
    lib.tri_prune_inplace.restype = i32
    if hasattr(lib, "tri_stamps_attach"):  # the measurement build only (include/tri_stamps.h)
        ip = ctypes.POINTER(ctypes.c_int)
        lib.tri_stamps_layout.argtypes = [ip, ip, ip]
        lib.tri_stamps_layout.restype = i32
        lib.tri_stamps_attach.argtypes = [vp]
        lib.tri_stamps_attach.restype = i32
    return lib


_lib = _load()


class TriError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {_lib.tri_status_string(status).decode()} (status {status})")


def _check(fn: str, status: int):
    if status != TRI_OK:
        raise TriError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    return t


def _key_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TRI_DT_BF16
    if t.dtype == torch.float32:
        return TRI_DT_F32
    raise TypeError("keys/values must be bfloat16 or float32")


# ---------------------------------------------------------------------------------------------

def tri_fold_weights(d: int, theta: float, offsets, centers=None):
    """Host fold: returns (W [F, 2] float64, mu [U, F, 2] float32 or None). ``centers`` is a
    host array [U, F, 2] (or [U, d] with interleaved pairs) of float32, or None."""
    offs = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    F = d // 2
    W = np.zeros((F, 2), dtype=np.float64)
    mu = None
    cptr, nu = None, 0
    if centers is not None:
        c = centers.numpy() if isinstance(centers, torch.Tensor) else np.asarray(centers)
        c = np.ascontiguousarray(c, dtype=np.float32).reshape(-1, F, 2)
        nu = c.shape[0]
        mu = np.zeros((nu, F, 2), dtype=np.float32)
        cptr = c.ctypes.data_as(ctypes.c_void_p)
    st = _lib.tri_fold_weights(int(d), float(theta), offs.ctypes.data_as(ctypes.c_void_p),
                               int(offs.size), cptr, int(nu), W.ctypes.data_as(ctypes.c_void_p),
                               None if mu is None else mu.ctypes.data_as(ctypes.c_void_p))
    _check("tri_fold_weights", st)
    return W, mu


def score_workspace_bytes(n_units: int) -> int:
    """Bytes of the histogram workspace tri_score alone needs."""
    n = ctypes.c_size_t(0)
    st = _lib.tri_score(None, TRI_DT_BF16, TRI_BANDS_INTERLEAVED, 128, 1.0, None, int(n_units), 0, 0,
                        None, None, None, None, None, ctypes.byref(n), None)
    _check("tri_score(query)", st)
    return int(n.value)


def workspace_bytes(n_units: int, max_rows: int) -> int:
    """Bytes of the workspace of tri_select_topb / tri_prune_pass (it also serves tri_score)."""
    n = ctypes.c_size_t(0)
    st = _lib.tri_select_topb(None, None, int(n_units), 0, int(max_rows), 0, None, None, None,
                              ctypes.byref(n), 0, None)
    _check("tri_select_topb(query)", st)
    return int(n.value)


def make_workspace(n_units: int, max_rows: int, device) -> torch.Tensor:
    """A workspace in its rest state (zero-filled once, at allocation)."""
    return torch.zeros(workspace_bytes(n_units, max_rows), dtype=torch.uint8, device=device)


def tri_score(keys: torch.Tensor, row_off: torch.Tensor, max_rows: int, pos: Optional[torch.Tensor],
              t_now: torch.Tensor, mu: torch.Tensor, theta: float, *,
              layout: int = TRI_BANDS_INTERLEAVED, scores: Optional[torch.Tensor] = None,
              ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Scores of every key; pos may be None when layout includes TRI_KEYS_ROTATED."""
    _dev(keys, "keys", ndim=2)
    dt = _key_dtype(keys)
    R, d = keys.shape
    _dev(row_off, "row_off", torch.int64, 1)
    U = row_off.numel() - 1
    if pos is not None or not (layout & TRI_KEYS_ROTATED):
        _dev(pos, "pos", torch.int32, 1)
        if pos.numel() != R:
            raise ValueError("pos has the wrong size")
    _dev(t_now, "t_now", torch.int32, 1)
    _dev(mu, "mu", torch.float32)
    if t_now.numel() != U or mu.numel() != U * d:
        raise ValueError("t_now or mu has the wrong size")
    if scores is None:
        scores = torch.empty(R, dtype=torch.float32, device=keys.device)
    _dev(scores, "scores", torch.float32, 1)
    if scores.numel() != R:
        raise ValueError("scores has the wrong size")
    wsp, nbytes = None, None
    if ws is not None:
        _dev(ws, "ws", torch.uint8, 1)
        wsp, nbytes = _ptr(ws), ctypes.byref(ctypes.c_size_t(ws.numel()))
    st = _lib.tri_score(_ptr(keys), dt, int(layout), int(d), float(theta), _ptr(row_off), int(U),
                        int(R), int(max_rows), _ptr(pos), _ptr(t_now), _ptr(mu), _ptr(scores),
                        wsp, nbytes, _stream(keys.device))
    _check("tri_score", st)
    return scores


def tri_score_max(keys: torch.Tensor, row_off: torch.Tensor, max_rows: int, pos: Optional[torch.Tensor],
                  t_now: torch.Tensor, centers: torch.Tensor, theta: float, offsets, *,
                  layout: int = TRI_BANDS_INTERLEAVED, scores: Optional[torch.Tensor] = None,
                  ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Maximum over the offset schedule of the unfolded score; centers are E[q] (device float32
    [U][d/2][2]), offsets a host sequence of ints. pos may be None with TRI_KEYS_ROTATED."""
    _dev(keys, "keys", ndim=2)
    dt = _key_dtype(keys)
    R, d = keys.shape
    _dev(row_off, "row_off", torch.int64, 1)
    U = row_off.numel() - 1
    if pos is not None:
        _dev(pos, "pos", torch.int32, 1)
        if pos.numel() != R:
            raise ValueError("pos has the wrong size")
    _dev(t_now, "t_now", torch.int32, 1)
    _dev(centers, "centers", torch.float32)
    if t_now.numel() != U or centers.numel() != U * d:
        raise ValueError("t_now or centers has the wrong size")
    offs = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    if scores is None:
        scores = torch.empty(R, dtype=torch.float32, device=keys.device)
    _dev(scores, "scores", torch.float32, 1)
    wsp, nbytes = None, None
    if ws is not None:
        _dev(ws, "ws", torch.uint8, 1)
        wsp, nbytes = _ptr(ws), ctypes.byref(ctypes.c_size_t(ws.numel()))
    st = _lib.tri_score_max(_ptr(keys), dt, int(layout), int(d), float(theta), offs.ctypes.data_as(ctypes.c_void_p),
                            int(offs.size), _ptr(row_off), int(U), int(R), int(max_rows), _ptr(pos), _ptr(t_now),
                            _ptr(centers), _ptr(scores), wsp, nbytes, _stream(keys.device))
    _check("tri_score_max", st)
    return scores


def tri_select_topb(scores: torch.Tensor, row_off: torch.Tensor, max_rows: int, B: int, *,
                    kept_idx: Optional[torch.Tensor] = None, kept_cnt: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None, hist_from_score: bool = False):
    _dev(scores, "scores", torch.float32, 1)
    _dev(row_off, "row_off", torch.int64, 1)
    U = row_off.numel() - 1
    dev = scores.device
    if kept_idx is None:
        kept_idx = torch.empty((U, B), dtype=torch.int32, device=dev)
    if kept_cnt is None:
        kept_cnt = torch.empty(U, dtype=torch.int32, device=dev)
    _dev(kept_idx, "kept_idx", torch.int32)
    _dev(kept_cnt, "kept_cnt", torch.int32, 1)
    if kept_idx.numel() != U * B or kept_cnt.numel() != U:
        raise ValueError("kept_idx or kept_cnt has the wrong size")
    if ws is None:
        if hist_from_score:
            raise ValueError("hist_from_score needs the workspace tri_score filled")
        ws = make_workspace(U, max_rows, dev)
    _dev(ws, "ws", torch.uint8, 1)
    wsp, nbytes = _ptr(ws), ctypes.byref(ctypes.c_size_t(ws.numel()))
    flags = TRI_SELECT_HIST_FROM_SCORE if hist_from_score else 0
    st = _lib.tri_select_topb(_ptr(scores), _ptr(row_off), int(U), int(scores.numel()), int(max_rows),
                              int(B), _ptr(kept_idx), _ptr(kept_cnt), wsp, nbytes, flags, _stream(dev))
    _check("tri_select_topb", st)
    return kept_idx, kept_cnt


def tri_compact_kv(K: torch.Tensor, V: torch.Tensor, pos: Optional[torch.Tensor], row_off: torch.Tensor,
                   kept_idx: torch.Tensor, kept_cnt: torch.Tensor, B: int, *,
                   K_out: Optional[torch.Tensor] = None, V_out: Optional[torch.Tensor] = None,
                   pos_out: Optional[torch.Tensor] = None):
    _dev(K, "K", ndim=2)
    _dev(V, "V", ndim=2)
    if V.dtype != K.dtype or V.shape != K.shape:
        raise ValueError("K and V must have the same dtype and shape")
    dt = _key_dtype(K)
    R, d = K.shape
    _dev(row_off, "row_off", torch.int64, 1)
    U = row_off.numel() - 1
    _dev(kept_idx, "kept_idx", torch.int32)
    _dev(kept_cnt, "kept_cnt", torch.int32, 1)
    dev = K.device
    if K_out is None:
        K_out = torch.zeros((U, B, d), dtype=K.dtype, device=dev)
    if V_out is None:
        V_out = torch.zeros((U, B, d), dtype=K.dtype, device=dev)
    _dev(K_out, "K_out", K.dtype)
    _dev(V_out, "V_out", K.dtype)
    if pos is not None:
        _dev(pos, "pos", torch.int32, 1)
        if pos_out is None:
            pos_out = torch.full((U, B), -1, dtype=torch.int32, device=dev)
        _dev(pos_out, "pos_out", torch.int32)
    if K_out.numel() != U * B * d or V_out.numel() != U * B * d:
        raise ValueError("K_out / V_out have the wrong size")
    st = _lib.tri_compact_kv(_ptr(K), _ptr(V), _ptr(pos), dt, int(d), _ptr(row_off), int(U), int(R),
                             _ptr(kept_idx), _ptr(kept_cnt), int(B), _ptr(K_out), _ptr(V_out),
                             _ptr(pos_out), _stream(dev))
    _check("tri_compact_kv", st)
    return K_out, V_out, pos_out


def _pass_args(K, V, pos, row_off, max_rows, t_now, mu, theta, B, ws, scores, kept_idx, kept_cnt,
               K_out, V_out, pos_out, layout, with_ws=True):
    _dev(K, "K", ndim=2)
    _dev(V, "V", ndim=2)
    if V.dtype != K.dtype or V.shape != K.shape:
        raise ValueError("K and V must have the same dtype and shape")
    dt = _key_dtype(K)
    R, d = K.shape
    dev = K.device
    _dev(row_off, "row_off", torch.int64, 1)
    U = row_off.numel() - 1
    _dev(pos, "pos", torch.int32, 1)
    _dev(t_now, "t_now", torch.int32, 1)
    _dev(mu, "mu", torch.float32)
    if pos.numel() != R or t_now.numel() != U or mu.numel() != U * d:
        raise ValueError("pos, t_now or mu has the wrong size")
    if ws is None and with_ws:
        ws = make_workspace(U, max_rows, dev)
    if scores is None:
        scores = torch.empty(R, dtype=torch.float32, device=dev)
    if kept_idx is None:
        kept_idx = torch.empty((U, B), dtype=torch.int32, device=dev)
    if kept_cnt is None:
        kept_cnt = torch.empty(U, dtype=torch.int32, device=dev)
    if K_out is None:
        K_out = torch.zeros((U, B, d), dtype=K.dtype, device=dev)
    if V_out is None:
        V_out = torch.zeros((U, B, d), dtype=K.dtype, device=dev)
    if pos_out is None:
        pos_out = torch.full((U, B), -1, dtype=torch.int32, device=dev)
    if with_ws:
        _dev(ws, "ws", torch.uint8, 1)
    _dev(scores, "scores", torch.float32, 1)
    _dev(kept_idx, "kept_idx", torch.int32)
    _dev(kept_cnt, "kept_cnt", torch.int32, 1)
    _dev(K_out, "K_out", K.dtype)
    _dev(V_out, "V_out", K.dtype)
    _dev(pos_out, "pos_out", torch.int32)
    if (scores.numel() != R or kept_idx.numel() != U * B or kept_cnt.numel() != U
            or K_out.numel() != U * B * d or V_out.numel() != U * B * d or pos_out.numel() != U * B):
        raise ValueError("an output has the wrong size")
    tensors = (K, V, pos, row_off, t_now, mu, ws, scores, kept_idx, kept_cnt, K_out, V_out, pos_out)
    args = (_ptr(K), _ptr(V), dt, int(layout), int(d), float(theta), _ptr(row_off), int(U), int(R),
            int(max_rows), _ptr(pos), _ptr(t_now), _ptr(mu), int(B), _ptr(scores), _ptr(kept_idx),
            _ptr(kept_cnt), _ptr(K_out), _ptr(V_out), _ptr(pos_out))
    if not with_ws:
        return tensors, None, args + (_stream(dev),)
    nbytes = ctypes.c_size_t(ws.numel())
    return tensors, nbytes, args + (_ptr(ws), ctypes.byref(nbytes), _stream(dev))


def prune_pass(K, V, pos, row_off, max_rows, t_now, mu, theta, B, *, ws=None, scores=None,
               kept_idx=None, kept_cnt=None, K_out=None, V_out=None, pos_out=None,
               layout=TRI_BANDS_INTERLEAVED):
    """One pruning pass through tri_prune_pass (score, select and compaction, three launches).
    Returns (scores, kept_idx, kept_cnt, K_out, V_out, pos_out)."""
    tensors, nbytes, args = _pass_args(K, V, pos, row_off, max_rows, t_now, mu, theta, B, ws, scores,
                                       kept_idx, kept_cnt, K_out, V_out, pos_out, layout)
    _check("tri_prune_pass", _lib.tri_prune_pass(*args))
    return tensors[7], tensors[8], tensors[9], tensors[10], tensors[11], tensors[12]


def prune_pass_max(K, V, pos, row_off, max_rows, t_now, centers, theta, offsets, B, *, ws=None, scores=None,
                   kept_idx=None, kept_cnt=None, K_out=None, V_out=None, pos_out=None,
                   layout=TRI_BANDS_INTERLEAVED):
    """One pruning pass with the maximum over the offsets as the score, through tri_prune_pass_max
    (centers: E[q] itself). Returns (scores, kept_idx, kept_cnt, K_out, V_out, pos_out)."""
    tensors, nbytes, args = _pass_args(K, V, pos, row_off, max_rows, t_now, centers, theta, B, ws, scores,
                                       kept_idx, kept_cnt, K_out, V_out, pos_out, layout)
    offs = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    args = args[:6] + (offs.ctypes.data_as(ctypes.c_void_p), int(offs.size)) + args[6:]
    _check("tri_prune_pass_max", _lib.tri_prune_pass_max(*args))
    return tensors[7], tensors[8], tensors[9], tensors[10], tensors[11], tensors[12]


def prune_pass_noalloc(K, V, pos, row_off, max_rows, t_now, mu, theta, B, *, scores=None, kept_idx=None,
                       kept_cnt=None, K_out=None, V_out=None, pos_out=None, layout=TRI_BANDS_INTERLEAVED):
    """The pruning pass through tri_prune_pass_noalloc: no workspace argument, the library's static
    device array instead (at most NOALLOC_SCRATCH_BYTES). Outputs not given are allocated here,
    by torch, before the call; the call itself allocates nothing.
    Returns (scores, kept_idx, kept_cnt, K_out, V_out, pos_out)."""
    tensors, _, args = _pass_args(K, V, pos, row_off, max_rows, t_now, mu, theta, B, None, scores, kept_idx,
                                  kept_cnt, K_out, V_out, pos_out, layout, with_ws=False)
    _check("tri_prune_pass_noalloc", _lib.tri_prune_pass_noalloc(*args))
    return tensors[7], tensors[8], tensors[9], tensors[10], tensors[11], tensors[12]


def prune_pass_3calls(K, V, pos, row_off, max_rows, t_now, mu, theta, B, *, ws=None, scores=None,
                      kept_idx=None, kept_cnt=None, K_out=None, V_out=None, pos_out=None,
                      layout=TRI_BANDS_INTERLEAVED):
    """The same pass as three separate calls: tri_score (histogram into ws), tri_select_topb
    (using that histogram) and tri_compact_kv."""
    U = row_off.numel() - 1
    if ws is None:
        ws = make_workspace(U, max_rows, K.device)
    scores = tri_score(K, row_off, max_rows, pos, t_now, mu, theta, layout=layout, scores=scores, ws=ws)
    kept_idx, kept_cnt = tri_select_topb(scores, row_off, max_rows, B, kept_idx=kept_idx,
                                         kept_cnt=kept_cnt, ws=ws, hist_from_score=True)
    K_out, V_out, pos_out = tri_compact_kv(K, V, pos, row_off, kept_idx, kept_cnt, B,
                                           K_out=K_out, V_out=V_out, pos_out=pos_out)
    return scores, kept_idx, kept_cnt, K_out, V_out, pos_out


def inplace_workspace_bytes(n_units: int, max_rows: int, B: int) -> int:
    """Bytes of the workspace of tri_prune_inplace."""
    n = ctypes.c_size_t(0)
    st = _lib.tri_prune_inplace(None, None, None, TRI_DT_BF16, TRI_BANDS_INTERLEAVED, 128, 1.0, None,
                                int(n_units), 0, int(max_rows), None, None, int(B), None, None, None,
                                ctypes.byref(n), None)
    _check("tri_prune_inplace(query)", st)
    return int(n.value)


def make_inplace_workspace(n_units: int, max_rows: int, B: int, device) -> torch.Tensor:
    """A tri_prune_inplace workspace in its rest state (zero-filled once, at allocation)."""
    return torch.zeros(inplace_workspace_bytes(n_units, max_rows, B), dtype=torch.uint8, device=device)


def _inplace_args(K, V, pos, row_off, max_rows, t_now, mu, theta, B, ws, scores, kept_cnt, layout):
    _dev(K, "K", ndim=2)
    dt = _key_dtype(K)
    R, d = K.shape
    _dev(V, "V", K.dtype, 2)
    if V.shape != K.shape:
        raise ValueError("V must have the shape of K")
    _dev(row_off, "row_off", torch.int64, 1)
    U = row_off.numel() - 1
    if pos is not None or not (layout & TRI_KEYS_ROTATED):
        _dev(pos, "pos", torch.int32, 1)
        if pos.numel() != R:
            raise ValueError("pos has the wrong size")
    _dev(t_now, "t_now", torch.int32, 1)
    _dev(mu, "mu", torch.float32)
    if t_now.numel() != U or mu.numel() != U * d:
        raise ValueError("t_now or mu has the wrong size")
    if ws is None:
        ws = make_inplace_workspace(U, max_rows, B, K.device)
    if scores is None:
        scores = torch.empty(R, dtype=torch.float32, device=K.device)
    if kept_cnt is None:
        kept_cnt = torch.empty(U, dtype=torch.int32, device=K.device)
    _dev(ws, "ws", torch.uint8, 1)
    _dev(scores, "scores", torch.float32, 1)
    _dev(kept_cnt, "kept_cnt", torch.int32, 1)
    if scores.numel() != R or kept_cnt.numel() != U:
        raise ValueError("scores or kept_cnt has the wrong size")
    tensors = (K, V, pos, row_off, t_now, mu, ws, scores, kept_cnt)
    nbytes = ctypes.c_size_t(ws.numel())
    args = (_ptr(K), _ptr(V), _ptr(pos), dt, int(layout), int(d), float(theta), _ptr(row_off), int(U), int(R),
            int(max_rows), _ptr(t_now), _ptr(mu), int(B), _ptr(scores), _ptr(kept_cnt), _ptr(ws),
            ctypes.byref(nbytes), _stream(K.device))
    return tensors, nbytes, args


def prune_inplace(K, V, pos, row_off, max_rows, t_now, mu, theta, B, *, ws=None, scores=None, kept_cnt=None,
                  layout=TRI_BANDS_INTERLEAVED):
    """tri_prune_inplace: prune every unit of the cache where it lives (K, V and pos are
    rewritten). Returns (scores, kept_cnt)."""
    tensors, nbytes, args = _inplace_args(K, V, pos, row_off, max_rows, t_now, mu, theta, B, ws, scores,
                                          kept_cnt, layout)
    _check("tri_prune_inplace", _lib.tri_prune_inplace(*args))
    return tensors[7], tensors[8]


class InplacePlan:
    """Arguments of tri_prune_inplace marshalled once, for repeated launches."""

    def __init__(self, K, V, pos, row_off, max_rows, t_now, mu, theta, B, *, ws, scores, kept_cnt,
                 layout=TRI_BANDS_INTERLEAVED):
        self._tensors, self._nbytes, self._args = _inplace_args(
            K, V, pos, row_off, max_rows, t_now, mu, theta, B, ws, scores, kept_cnt, layout)

    def run(self):
        _check("tri_prune_inplace", _lib.tri_prune_inplace(*self._args))


class MaxPassPlan:
    """The max-over-offsets pass with arguments marshalled once: run() is tri_prune_pass_max (ws
    sized as for tri_prune_pass), run3() the same pass as three calls (tri_score_max with its
    histogram into ws, tri_select_topb on that histogram, tri_compact_kv), score() the score alone."""

    def __init__(self, K, V, pos, row_off, max_rows, t_now, centers, theta, offsets, B, *, ws, scores,
                 kept_idx, kept_cnt, K_out, V_out, pos_out, layout=TRI_BANDS_INTERLEAVED):
        _dev(K, "K", ndim=2)
        dt = _key_dtype(K)
        R, d = K.shape
        U = row_off.numel() - 1
        for t, name in [(V, "V"), (K_out, "K_out"), (V_out, "V_out")]:
            _dev(t, name, K.dtype)
        for t, name in [(pos, "pos"), (t_now, "t_now"), (kept_idx, "kept_idx"), (kept_cnt, "kept_cnt"),
                        (pos_out, "pos_out")]:
            _dev(t, name, torch.int32)
        _dev(row_off, "row_off", torch.int64, 1)
        _dev(centers, "centers", torch.float32)
        _dev(scores, "scores", torch.float32, 1)
        _dev(ws, "ws", torch.uint8, 1)
        if (V.shape != K.shape or pos.numel() != R or t_now.numel() != U or centers.numel() != U * d
                or scores.numel() != R or kept_idx.numel() != U * B or kept_cnt.numel() != U
                or K_out.numel() != U * B * d or V_out.numel() != U * B * d or pos_out.numel() != U * B):
            raise ValueError("a tensor has the wrong size")
        self._offs = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
        self._nbytes = ctypes.c_size_t(ws.numel())
        self._tensors = (K, V, pos, row_off, t_now, centers, ws, scores, kept_idx, kept_cnt, K_out, V_out, pos_out)
        st = _stream(K.device)
        nb = ctypes.byref(self._nbytes)
        self._score = (_ptr(K), dt, int(layout), int(d), float(theta), self._offs.ctypes.data_as(ctypes.c_void_p),
                       int(self._offs.size), _ptr(row_off), int(U), int(R), int(max_rows), _ptr(pos), _ptr(t_now),
                       _ptr(centers), _ptr(scores), _ptr(ws), nb, st)
        self._select = (_ptr(scores), _ptr(row_off), int(U), int(R), int(max_rows), int(B), _ptr(kept_idx),
                        _ptr(kept_cnt), _ptr(ws), nb, TRI_SELECT_HIST_FROM_SCORE, st)
        self._compact = (_ptr(K), _ptr(V), _ptr(pos), dt, int(d), _ptr(row_off), int(U), int(R), _ptr(kept_idx),
                         _ptr(kept_cnt), int(B), _ptr(K_out), _ptr(V_out), _ptr(pos_out), st)
        self._fused = (_ptr(K), _ptr(V), dt, int(layout), int(d), float(theta),
                       self._offs.ctypes.data_as(ctypes.c_void_p), int(self._offs.size), _ptr(row_off), int(U),
                       int(R), int(max_rows), _ptr(pos), _ptr(t_now), _ptr(centers), int(B), _ptr(scores),
                       _ptr(kept_idx), _ptr(kept_cnt), _ptr(K_out), _ptr(V_out), _ptr(pos_out), _ptr(ws), nb, st)

    def score(self):
        _check("tri_score_max", _lib.tri_score_max(*self._score))

    def run(self):
        _check("tri_prune_pass_max", _lib.tri_prune_pass_max(*self._fused))

    def run3(self):
        _check("tri_score_max", _lib.tri_score_max(*self._score))
        _check("tri_select_topb", _lib.tri_select_topb(*self._select))
        _check("tri_compact_kv", _lib.tri_compact_kv(*self._compact))


class ScorePlan:
    """Arguments of tri_score marshalled once, for repeated launches with little host overhead
    (used to time the score kernel alone). With ws, every launch adds its histogram into ws."""

    def __init__(self, keys, row_off, max_rows, pos, t_now, mu, theta, *, scores, ws=None,
                 layout=TRI_BANDS_INTERLEAVED):
        _dev(keys, "keys", ndim=2)
        dt = _key_dtype(keys)
        R, d = keys.shape
        _dev(row_off, "row_off", torch.int64, 1)
        U = row_off.numel() - 1
        if pos is not None or not (layout & TRI_KEYS_ROTATED):
            _dev(pos, "pos", torch.int32, 1)
            if pos.numel() != R:
                raise ValueError("pos has the wrong size")
        _dev(t_now, "t_now", torch.int32, 1)
        _dev(mu, "mu", torch.float32)
        _dev(scores, "scores", torch.float32, 1)
        if t_now.numel() != U or mu.numel() != U * d or scores.numel() != R:
            raise ValueError("t_now, mu or scores has the wrong size")
        wsp, self._nbytes = None, None
        if ws is not None:
            _dev(ws, "ws", torch.uint8, 1)
            self._nbytes = ctypes.c_size_t(ws.numel())
            wsp = _ptr(ws)
        self._tensors = (keys, row_off, pos, t_now, mu, scores, ws)
        self._args = (_ptr(keys), dt, int(layout), int(d), float(theta), _ptr(row_off), int(U), int(R),
                      int(max_rows), _ptr(pos), _ptr(t_now), _ptr(mu), _ptr(scores), wsp,
                      None if ws is None else ctypes.byref(self._nbytes), _stream(keys.device))

    def run(self):
        _check("tri_score", _lib.tri_score(*self._args))


class PassPlan:
    """Arguments of tri_prune_pass marshalled once, for repeated launches with little host
    overhead. The tensors are held by the plan; launches go to the stream current at
    construction."""

    def __init__(self, K, V, pos, row_off, max_rows, t_now, mu, theta, B, *, ws, scores, kept_idx,
                 kept_cnt, K_out, V_out, pos_out, layout=TRI_BANDS_INTERLEAVED):
        self._tensors, self._nbytes, self._args = _pass_args(
            K, V, pos, row_off, max_rows, t_now, mu, theta, B, ws, scores, kept_idx, kept_cnt,
            K_out, V_out, pos_out, layout)

    def run(self):
        _check("tri_prune_pass", _lib.tri_prune_pass(*self._args))


def stamps_layout():
    """(workgroups, points, kernels) of the timestamp buffer of the measurement build
    (include/tri_stamps.h); raises when the loaded library has no stamps."""
    if not hasattr(_lib, "tri_stamps_layout"):
        raise RuntimeError(f"{_LIB_PATH} has no timestamps: build libtri_stamps.so with "
                           "`python -m rotary_frequency_key_amd.build --stamps` and load it through TRI_LIBRARY")
    w, p, k = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check("tri_stamps_layout", _lib.tri_stamps_layout(ctypes.byref(w), ctypes.byref(p), ctypes.byref(k)))
    return w.value, p.value, k.value


def stamps_attach(buf: Optional[torch.Tensor]):
    """Attach a zeroed int64 device tensor of kernels * workgroups * points entries as the
    timestamp buffer (None detaches)."""
    w, p, k = stamps_layout()
    if buf is not None:
        if buf.dtype != torch.int64 or not buf.is_cuda or buf.numel() != w * p * k or not buf.is_contiguous():
            raise ValueError(f"the stamp buffer must be a contiguous int64 device tensor of {k * w * p} entries")
    _check("tri_stamps_attach", _lib.tri_stamps_attach(_ptr(buf)))
