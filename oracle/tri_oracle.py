"""Plain fp64 reference for the offset-averaged trigonometric key score, top-B select and
K/V compaction.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``. It shares no code with the HIP library and imports
nothing from it. Everything is NumPy fp64 over whole arrays of one unit (one KV head of one
layer of one sequence); no blocking, fusion or reordering beyond what each formula states.

Page cited throughout: "The future-offset average in TriAttention can be precomputed"
(A. Mukherjee), hereafter "the note".

Readings of points the note leaves open (each one is used below):
  R1  band f of a d-vector x is the complex number x[2f] + i*x[2f+1] (interleaved pairs,
      the rotary pairing of RoFormer that the note invokes when it reads a pair as one
      complex number). The half-split storage x[f] + i*x[f+d/2] is a second layout.
  R2  the query-key distance is delta = t - p (current position minus key position), and a
      future offset d adds to it, delta + d.
  R3  S_norm is omitted: the note sets it aside and never defines it.
  R4  D is {2^0, ..., 2^16}: 17 offsets, 1 included, 0 excluded.
  R9  ties in the score keep the lower row index; -0.0 and +0.0 are equal.
  R10 a NaN score ranks below every number (finite inputs are a precondition).
  R11 the budget B applies to each unit; B >= N keeps every row, B = 0 keeps none.
  R12 kept rows are emitted in ascending original row order.

Parity status per function (what pins it is in tests/test_oracle_pins.py):
  rotary_frequencies, power_of_two_offsets, as_bands, widen_bf16  pinned
  score_unfolded, fold_weights, fold_weights_real, folded_center,
  score_folded_complex, score_folded_polar, score_folded_real       pinned
  score_unfolded_max                                                 pinned
  score_post_rope                                                    pinned
  select_topb                                                        pinned
  compact_rows                                                       pinned
No function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rotary_frequencies",
    "power_of_two_offsets",
    "widen_bf16",
    "as_bands",
    "distances",
    "score_unfolded",
    "score_unfolded_max",
    "fold_weights",
    "fold_weights_real",
    "folded_center",
    "score_folded_complex",
    "score_folded_polar",
    "score_folded_real",
    "score_post_rope",
    "rotate_keys",
    "select_topb",
    "compact_rows",
    "unit_pass",
]


# ---------------------------------------------------------------------------------------------
# Constants of the score
# ---------------------------------------------------------------------------------------------

def rotary_frequencies(d: int, theta: float) -> np.ndarray:
    """omega_f = theta^(-2f/d) for f = 0 .. d/2-1, in fp64.

    The note, section "The score TriAttention computes": band f turns at angular frequency
    theta^(-2f/d) with rotary base theta (10000 on the page; each workload names its own).
    """
    if d <= 0 or d % 2:
        raise ValueError("d must be a positive even number")
    f = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * f / d)


def power_of_two_offsets() -> np.ndarray:
    """The future-offset schedule D = {1, 2, 4, ..., 2^16} (17 offsets).

    The note, section "The averaging step" (the set D) and its introduction (powers of two
    from 2^0 to 2^16). Reading R4.
    """
    return np.array([1 << j for j in range(17)], dtype=np.int64)


# ---------------------------------------------------------------------------------------------
# Inputs
# ---------------------------------------------------------------------------------------------

def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact fp64 values.

    A bfloat16 is the top half of an IEEE binary32, so shifting its 16 bits into the high
    half of a 32-bit word gives the binary32 with the same value; binary32 -> binary64 is exact.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_bands(x: np.ndarray, layout: str = "interleaved") -> np.ndarray:
    """Read the last axis (length d) of a real array as d/2 complex bands.

    The note, section "The same score, read as arrows in the plane": a rotary pair is a point
    in the plane, i.e. one complex number. Reading R1 fixes which coordinates pair up.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("last axis must have even length")
    if layout == "interleaved":
        return x[..., 0::2] + 1j * x[..., 1::2]
    if layout == "half_split":
        return x[..., : d // 2] + 1j * x[..., d // 2:]
    raise ValueError(f"unknown layout {layout!r}")


def distances(t_now: int, pos: np.ndarray) -> np.ndarray:
    """Query-key distance delta = t - p per key, as exact int64 (reading R2).

    The note, section "The score TriAttention computes": the only varying quantity left in the
    logit is the query-key distance.
    """
    return np.int64(t_now) - np.asarray(pos, dtype=np.int64)


# ---------------------------------------------------------------------------------------------
# Scores
# ---------------------------------------------------------------------------------------------

def _count(counter, key, n):
    if counter is not None:
        counter[key] = counter.get(key, 0) + int(n)


def score_unfolded(center, keys, delta, omega, offsets, counter=None) -> np.ndarray:
    """Literal offset average of the polar trigonometric score, one offset at a time.

    S(k, D')   = sum_f |E[q_f]| |k_f| cos(omega_f * D' + phi_f),  phi_f = arg E[q_f] - arg k_f
    S~(k)      = (1/|D|) sum_{d in D} S(k, delta + d)

    The note: section "The score TriAttention computes" (polar form and the definition of
    phi_f) and section "The averaging step" (the offset average). This is the per-offset
    evaluation the note describes for the original implementation, looping over offsets
    instead of materialising the [keys x offsets x bands] table.

    center: complex [F]; keys: complex [N, F]; delta: int [N]; omega: [F]; offsets: int [|D|].
    ``counter['band_cos']`` (if given) counts band-cosine evaluations.
    """
    center = np.asarray(center, dtype=np.complex128)
    keys = np.asarray(keys, dtype=np.complex128)
    delta = np.asarray(delta, dtype=np.int64)
    amp = np.abs(center)[None, :] * np.abs(keys)
    phi = np.angle(center)[None, :] - np.angle(keys)
    total = np.zeros(keys.shape[0], dtype=np.float64)
    for off in np.asarray(offsets, dtype=np.int64):
        dist = (delta + off).astype(np.float64)  # exact: integers far below 2^53
        total += np.sum(amp * np.cos(omega[None, :] * dist[:, None] + phi), axis=1)
        _count(counter, "band_cos", keys.size)
    return total / len(offsets)


def score_unfolded_max(center, keys, delta, omega, offsets, counter=None) -> np.ndarray:
    """Max-over-offsets variant: max_{d in D} S(k, delta + d), S the polar score above.

    The note, section "What it saves, and what it does not": a non-default variant takes a
    maximum over the offsets instead of the mean; it is not linear, so it does not fold.
    """
    center = np.asarray(center, dtype=np.complex128)
    keys = np.asarray(keys, dtype=np.complex128)
    delta = np.asarray(delta, dtype=np.int64)
    amp = np.abs(center)[None, :] * np.abs(keys)
    phi = np.angle(center)[None, :] - np.angle(keys)
    best = np.full(keys.shape[0], -np.inf, dtype=np.float64)
    for off in np.asarray(offsets, dtype=np.int64):
        dist = (delta + off).astype(np.float64)
        best = np.maximum(best, np.sum(amp * np.cos(omega[None, :] * dist[:, None] + phi), axis=1))
        _count(counter, "band_cos", keys.size)
    return best


def fold_weights(omega, offsets, counter=None) -> np.ndarray:
    """W_f = (1/|D|) sum_{d in D} e^{i omega_f d}, complex [F].

    The note, section "The averaging step": the offset factor of the rotation collapses into
    one complex weight per band, depending only on the frequencies and the offset set.
    """
    omega = np.asarray(omega, dtype=np.float64)
    offs = np.asarray(offsets, dtype=np.int64).astype(np.float64)
    _count(counter, "weight_exp", omega.size * offs.size)
    return np.exp(1j * omega[:, None] * offs[None, :]).sum(axis=1) / offs.size


def fold_weights_real(omega, offsets):
    """(Re W_f, Im W_f) computed with real cosines and sines only:
    Re W_f = (1/|D|) sum_d cos(omega_f d),  Im W_f = (1/|D|) sum_d sin(omega_f d).

    The same weight as ``fold_weights`` (the note, section "The averaging step"), written in the
    real arithmetic of the real-coefficient form.
    """
    omega = np.asarray(omega, dtype=np.float64)
    offs = np.asarray(offsets, dtype=np.int64).astype(np.float64)
    ang = omega[:, None] * offs[None, :]
    return np.cos(ang).sum(axis=1) / offs.size, np.sin(ang).sum(axis=1) / offs.size


def folded_center(center, weights) -> np.ndarray:
    """mu'_f = E[q_f] * W_f: the offset-averaged center (the note, section "The averaging
    step", the folded polar equation)."""
    return np.asarray(center, dtype=np.complex128) * np.asarray(weights, dtype=np.complex128)


def score_folded_complex(mu, keys, delta, omega, counter=None) -> np.ndarray:
    """S~(k) = Re{ sum_f mu'_f * conj(k_f) * e^{i omega_f delta} }.

    The note, section "The averaging step": the offset average as one evaluation of the
    complex (RoFormer) form with the center replaced by mu' = E[q] W.
    """
    mu = np.asarray(mu, dtype=np.complex128)
    keys = np.asarray(keys, dtype=np.complex128)
    dist = np.asarray(delta, dtype=np.int64).astype(np.float64)
    rot = np.exp(1j * omega[None, :] * dist[:, None])
    _count(counter, "band_cos", keys.size)
    return np.real(np.sum(mu[None, :] * np.conj(keys) * rot, axis=1))


def score_folded_polar(mu, keys, delta, omega) -> np.ndarray:
    """S~(k) = sum_f |mu'_f| |k_f| cos(omega_f delta + phi'_f), phi'_f = arg mu'_f - arg k_f.

    The note, section "The averaging step", the folded polar equation.
    """
    mu = np.asarray(mu, dtype=np.complex128)
    keys = np.asarray(keys, dtype=np.complex128)
    dist = np.asarray(delta, dtype=np.int64).astype(np.float64)
    amp = np.abs(mu)[None, :] * np.abs(keys)
    phi = np.angle(mu)[None, :] - np.angle(keys)
    return np.sum(amp * np.cos(omega[None, :] * dist[:, None] + phi), axis=1)


def score_folded_real(center_xy, w_re, w_im, key_xy, delta, omega) -> np.ndarray:
    """Real-coefficient form, no complex numbers.

    The note, section "The averaging step", last paragraph: W_f folds into the real cosine and
    sine coefficients as a fixed 2x2 map per band. With band pairs (x, y) read as in R1:
      center pair (qx, qy) -> (a qx - b qy, b qx + a qy)           [W_f = a + ib, the 2x2 map]
      cos coefficient  A_f = cx kx + cy ky
      sin coefficient  B_f = cy kx - cx ky
      S~(k) = sum_f A_f cos(omega_f delta) - B_f sin(omega_f delta)

    center_xy: real [d] (interleaved pairs); key_xy: real [N, d]; w_re, w_im: real [F].
    """
    c = np.asarray(center_xy, dtype=np.float64)
    k = np.asarray(key_xy, dtype=np.float64)
    qx, qy = c[0::2], c[1::2]
    kx, ky = k[:, 0::2], k[:, 1::2]
    cx = w_re * qx - w_im * qy
    cy = w_im * qx + w_re * qy
    a_coef = cx[None, :] * kx + cy[None, :] * ky
    b_coef = cy[None, :] * kx - cx[None, :] * ky
    ang = omega[None, :] * np.asarray(delta, dtype=np.int64).astype(np.float64)[:, None]
    return np.sum(a_coef * np.cos(ang) - b_coef * np.sin(ang), axis=1)


def rotate_keys(keys, pos, omega) -> np.ndarray:
    """Post-rotation keys: k_f * e^{i omega_f p} per key (the rotation is a multiplication,
    the note, section "The same score, read as arrows in the plane")."""
    p = np.asarray(pos, dtype=np.int64).astype(np.float64)
    return np.asarray(keys, dtype=np.complex128) * np.exp(1j * omega[None, :] * p[:, None])


def score_post_rope(mu, rotated_keys, t_now, omega) -> np.ndarray:
    """The same S~ for keys stored after rotation (k^rot_f = k_f e^{i omega_f p}):
    S~(k) = Re{ sum_f (mu'_f e^{i omega_f t}) * conj(k^rot_f) }.

    Follows from the factorisation of rotations in the note, section "The averaging step"
    (e^{i w (t - p)} = e^{i w t} e^{-i w p}), applied to the folded complex form.
    """
    coef = np.asarray(mu, dtype=np.complex128) * np.exp(1j * omega * np.float64(t_now))
    return np.real(np.sum(coef[None, :] * np.conj(np.asarray(rotated_keys, dtype=np.complex128)), axis=1))


# ---------------------------------------------------------------------------------------------
# Select and compaction
# ---------------------------------------------------------------------------------------------

def select_topb(scores, budget: int) -> np.ndarray:
    """Kept row indices of one unit, ascending (R12).

    The note, introduction: when the cache must be trimmed, keys are scored and the highest-
    scoring ones are kept; the README's KV budget bounds how many (R11). Order: score
    descending, then row index ascending (R9); -0 == +0; NaN below every number (R10).
    Keeps min(budget, N) rows.
    """
    s = np.asarray(scores, dtype=np.float64) + 0.0  # -0.0 + 0.0 == +0.0
    n = s.size
    if budget < 0:
        raise ValueError("budget must be >= 0")
    is_nan = np.isnan(s)
    neg = np.where(is_nan, 0.0, -s)
    order = np.lexsort((np.arange(n), neg, is_nan))  # last key is the primary one
    return np.sort(order[: min(budget, n)]).astype(np.int64)


def compact_rows(rows: np.ndarray, kept: np.ndarray, budget: int, fill) -> np.ndarray:
    """Dense copy of the kept rows: out[j] = rows[kept[j]] for j < len(kept); rows j >= len(kept)
    of the [budget, ...] output keep ``fill``. A byte copy: dtype and bits are preserved.

    The note, introduction: the pruned cache. README: compressed cache entries.
    """
    rows = np.asarray(rows)
    out = np.empty((budget,) + rows.shape[1:], dtype=rows.dtype)
    out[...] = fill
    for j, src in enumerate(np.asarray(kept, dtype=np.int64)):
        out[j] = rows[src]
    return out


# ---------------------------------------------------------------------------------------------
# One unit end to end
# ---------------------------------------------------------------------------------------------

def unit_pass(center_f32, keys, values, pos, t_now, d, theta, offsets, budget,
              key_dtype="bf16", layout="interleaved"):
    """Score (folded complex form), select and compact one unit, from the exact input bits.

    center_f32: float32 [d]; keys, values: uint16 bf16 bits or float32, [N, d]; pos: int [N].
    Returns dict(scores, kept, K_out, V_out, pos_out) with unfilled output rows zero / -1.
    """
    omega = rotary_frequencies(d, theta)
    if key_dtype == "bf16":
        k_real = widen_bf16(keys)
    else:
        k_real = np.asarray(keys, dtype=np.float32).astype(np.float64)
    center = as_bands(np.asarray(center_f32, dtype=np.float32).astype(np.float64), layout)
    kb = as_bands(k_real, layout)
    mu = folded_center(center, fold_weights(omega, offsets))
    scores = score_folded_complex(mu, kb, distances(t_now, pos), omega)
    kept = select_topb(scores, budget)
    zero = np.zeros((), dtype=np.asarray(keys).dtype)
    return {
        "scores": scores,
        "kept": kept,
        "K_out": compact_rows(keys, kept, budget, zero),
        "V_out": compact_rows(values, kept, budget, zero),
        "pos_out": compact_rows(np.asarray(pos, dtype=np.int32), kept, budget, np.int32(-1)),
    }
