"""Pins of the fp64 oracle against what the note and the mathematics fix, independently of the
oracle's own formulas: textbook rotary rotation matrices, closed forms of geometric sums,
brute-force subset enumeration, invariants and special cases.

Page: "The future-offset average in TriAttention can be precomputed" (the note).
Tolerances use the scaled error e = |a - b| / max(|b|, L1/F), L1 = sum_f |mu'_f||k_f| (the mean
per-band term magnitude sets the scale of a score whose terms cancel).
"""
import itertools
import math

import numpy as np
import pytest

import oracle as O
from synthgen import f32_to_bf16_bits, pack_units, unit_inputs, workload


def scaled_err(a, b, scale):
    return np.abs(np.asarray(a) - np.asarray(b)) / np.maximum(np.abs(np.asarray(b)), scale)


def l1_scale(mu, kb):
    return np.sum(np.abs(mu)[None, :] * np.abs(kb), axis=1) / kb.shape[1]


def rope_rotate(x, pos, omega):
    """Textbook rotary embedding of real vectors x [N, d] at positions pos [N]: each coordinate
    pair (x[2f], x[2f+1]) is multiplied by the 2x2 rotation matrix of angle omega_f * pos
    (counter-clockwise), written out with real cos/sin and matrices, no complex numbers."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    for f in range(x.shape[1] // 2):
        ang = omega[f] * np.asarray(pos, dtype=np.float64)
        c, s = np.cos(ang), np.sin(ang)
        for i in range(x.shape[0]):
            rot = np.array([[c[i], -s[i]], [s[i], c[i]]])
            out[i, 2 * f:2 * f + 2] = rot @ x[i, 2 * f:2 * f + 2]
    return out


def small_case(seed=0, n=24, d=16, theta=1e4):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(d) * 2.0
    k = rng.standard_normal(d)[None, :] * 2.0 + 0.5 * rng.standard_normal((n, d))
    pos = rng.integers(0, 5000, size=n)
    t = 5000
    return q, k, pos, t, O.rotary_frequencies(d, theta)


# --------------------------------------------------------------------------------------------
# Constants
# --------------------------------------------------------------------------------------------

def test_rotary_frequency_closed_values():
    # omega_0 = 1 for any base; omega_{d/4} = theta^(-1/2); constant ratio theta^(-2/d).
    for d, theta in [(128, 1e4), (128, 1e6), (64, 5e5), (256, 1e4)]:
        w = O.rotary_frequencies(d, theta)
        assert w.shape == (d // 2,)
        assert w[0] == 1.0
        assert math.isclose(w[d // 4], 1.0 / math.sqrt(theta), rel_tol=1e-14)
        ratios = w[1:] / w[:-1]
        assert np.allclose(ratios, theta ** (-2.0 / d), rtol=1e-13, atol=0)
        assert np.all(np.diff(w) < 0)
    assert math.isclose(O.rotary_frequencies(128, 1e4)[32], 0.01, rel_tol=1e-14)


def test_offset_schedule():
    D = O.power_of_two_offsets()
    assert D.tolist() == [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192,
                          16384, 32768, 65536]


def test_bf16_rounding_and_widening():
    import torch
    vals = np.array([1.0, -2.5, 3.14159265, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -0.0, 1e-30, 65504.0,
                     0.1, -7.77e10], dtype=np.float32)
    bits = f32_to_bf16_bits(vals)
    assert bits[0] == 0x3F80 and bits[3] == 0x3F80 and bits[4] == 0x3F82  # ties to even
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    rnd = np.random.default_rng(7).standard_normal(100000).astype(np.float32) * 10
    ref = torch.from_numpy(rnd).to(torch.bfloat16)
    assert np.array_equal(f32_to_bf16_bits(rnd), ref.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(O.widen_bf16(f32_to_bf16_bits(rnd)), ref.to(torch.float64).numpy())
    assert O.widen_bf16(np.array([0x4049], dtype=np.uint16))[0] == 3.140625


def test_band_layouts():
    x = np.arange(8, dtype=np.float64)
    assert np.array_equal(O.as_bands(x), np.array([0 + 1j, 2 + 3j, 4 + 5j, 6 + 7j]))
    assert np.array_equal(O.as_bands(x, "half_split"), np.array([0 + 4j, 1 + 5j, 2 + 6j, 3 + 7j]))


# --------------------------------------------------------------------------------------------
# Fold weights: closed forms and invariants
# --------------------------------------------------------------------------------------------

def test_fold_weight_geometric_closed_form():
    # For D = {0, 1, ..., M-1}: W = (1/M) (1 - e^{i w M}) / (1 - e^{i w}) (geometric series),
    # |W| = |sin(M w / 2) / (M sin(w / 2))| (Dirichlet kernel).
    omega = np.array([0.3, 1.0, 2.0, 0.01, 2.9])
    for M in [1, 2, 5, 17, 100]:
        D = np.arange(M)
        W = O.fold_weights(omega, D)
        closed = (1 - np.exp(1j * omega * M)) / (1 - np.exp(1j * omega)) / M
        assert np.allclose(W, closed, atol=1e-14, rtol=0)
        assert np.allclose(np.abs(W), np.abs(np.sin(M * omega / 2) / (M * np.sin(omega / 2))),
                           atol=1e-14)
        wr, wi = O.fold_weights_real(omega, D)
        assert np.allclose(wr, closed.real, atol=1e-14) and np.allclose(wi, closed.imag, atol=1e-14)


def test_fold_weight_invariants():
    D = O.power_of_two_offsets()
    for d, theta in [(128, 1e4), (128, 1e6), (128, 5e5)]:
        w = O.rotary_frequencies(d, theta)
        W = O.fold_weights(w, D)
        assert np.all(np.abs(W) <= 1 + 1e-15)
        # conjugate symmetry
        assert np.allclose(O.fold_weights(-w, D), np.conj(W), atol=1e-15)
        # slow bands: every offset turns by almost nothing, W -> 1
        slow = w * D.max() < 1e-2
        assert np.all(np.abs(W[slow] - 1) < w[slow] * D.max())
    # D = {0}: no averaging, W = 1 exactly
    assert np.all(O.fold_weights(O.rotary_frequencies(128, 1e6), [0]) == 1)
    # omega * d a multiple of 2 pi for every offset -> W = 1
    assert np.allclose(O.fold_weights(np.array([2 * np.pi, 4 * np.pi]), D), 1, atol=1e-9)
    # band 0 turns at 1 rad per position whatever the base: its weight is the same for all bases
    W0 = [O.fold_weights(O.rotary_frequencies(d, th), D)[0] for d, th in [(128, 1e4), (64, 1e6)]]
    assert W0[0] == W0[1]
    # high-frequency bands cancel, low-frequency bands reinforce (the note's second figure)
    W = O.fold_weights(O.rotary_frequencies(128, 1e6), D)
    assert abs(W[0]) < 0.2 and abs(W[-1]) > 0.99


# --------------------------------------------------------------------------------------------
# Scores against textbook rotary attention
# --------------------------------------------------------------------------------------------

def test_single_offset_is_rope_logit():
    # D = {0}: the averaged score is the rotary attention logit <R(t) q, R(p) k> of the
    # center and the key; rotation written with real matrices (RoFormer's definition).
    q, k, pos, t, omega = small_case(1)
    ref = rope_rotate(np.repeat(q[None, :], len(pos), 0), np.full(len(pos), t), omega)
    ref = np.sum(ref * rope_rotate(k, pos, omega), axis=1)
    qb, kb = O.as_bands(q), O.as_bands(k)
    delta = O.distances(t, pos)
    mu = O.folded_center(qb, O.fold_weights(omega, [0]))
    for got in [O.score_unfolded(qb, kb, delta, omega, [0]),
                O.score_folded_complex(mu, kb, delta, omega),
                O.score_folded_polar(mu, kb, delta, omega),
                O.score_folded_real(q, *O.fold_weights_real(omega, [0]), k, delta, omega)]:
        assert np.max(scaled_err(got, ref, l1_scale(qb, kb))) < 1e-12


def test_offset_average_is_mean_of_future_rope_logits():
    # The offset average is the mean over d in D of the logit of the center rotated to t + d
    # and the key rotated to p (reading R2), computed with rotation matrices.
    q, k, pos, t, omega = small_case(2, n=12, d=8)
    D = O.power_of_two_offsets()
    kr = rope_rotate(k, pos, omega)
    ref = np.zeros(len(pos))
    for off in D:
        qr = rope_rotate(np.repeat(q[None, :], len(pos), 0), np.full(len(pos), t + off), omega)
        ref += np.sum(qr * kr, axis=1)
    ref /= len(D)
    qb, kb = O.as_bands(q), O.as_bands(k)
    delta = O.distances(t, pos)
    W = O.fold_weights(omega, D)
    mu = O.folded_center(qb, W)
    scale = l1_scale(mu, kb)
    assert np.max(scaled_err(O.score_unfolded(qb, kb, delta, omega, D), ref, scale)) < 1e-11
    assert np.max(scaled_err(O.score_folded_complex(mu, kb, delta, omega), ref, scale)) < 1e-11
    # a sign slip in the distance (p - t) would not match
    wrong = O.score_folded_complex(mu, kb, -delta, omega)
    assert np.max(scaled_err(wrong, ref, scale)) > 1e-2


def test_half_split_layout_is_a_permutation():
    q, k, pos, t, omega = small_case(3)
    d = q.size
    perm = np.empty(d, dtype=int)  # interleaved index -> half-split index
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    qh, kh = np.empty_like(q), np.empty_like(k)
    qh[perm], kh[:, perm] = q, k
    D = O.power_of_two_offsets()
    W = O.fold_weights(omega, D)
    a = O.score_folded_complex(O.folded_center(O.as_bands(q), W), O.as_bands(k), t - pos, omega)
    b = O.score_folded_complex(O.folded_center(O.as_bands(qh, "half_split"), W),
                               O.as_bands(kh, "half_split"), t - pos, omega)
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------------------------
# The fold is exact (P1, P2) and costs a factor |D| less (P10)
# --------------------------------------------------------------------------------------------

def _c1_unit():
    wl = workload("c1")
    inp = unit_inputs(wl, 0)
    omega = O.rotary_frequencies(wl.d, wl.theta)
    qb = O.as_bands(inp["center"].astype(np.float64))
    kb = O.as_bands(inp["keys"].astype(np.float64))
    return wl, inp, omega, qb, kb, O.distances(inp["t"], inp["pos"])


def test_fold_matches_literal_offset_loop_c1():
    wl, inp, omega, qb, kb, delta = _c1_unit()
    D = O.power_of_two_offsets()
    W = O.fold_weights(omega, D)
    mu = O.folded_center(qb, W)
    scale = l1_scale(mu, kb)
    lit = O.score_unfolded(qb, kb, delta, omega, D)
    forms = {
        "complex": O.score_folded_complex(mu, kb, delta, omega),
        "polar": O.score_folded_polar(mu, kb, delta, omega),
        "real2x2": O.score_folded_real(inp["center"].astype(np.float64), *O.fold_weights_real(omega, D),
                                       inp["keys"].astype(np.float64), delta, omega),
    }
    for name, s in forms.items():
        e = np.max(scaled_err(s, lit, scale))
        assert e < 1e-9, (name, e)
    # the mean is the mean: leaving out the 1/|D| (or an offset) is caught
    assert np.max(scaled_err(O.score_unfolded(qb, kb, delta, omega, D[:-1]), lit, scale)) > 1e-3


def test_fold_preserves_ranking_c1():
    wl, inp, omega, qb, kb, delta = _c1_unit()
    D = O.power_of_two_offsets()
    mu = O.folded_center(qb, O.fold_weights(omega, D))
    lit = O.score_unfolded(qb, kb, delta, omega, D)
    fold = O.score_folded_complex(mu, kb, delta, omega)
    scale = l1_scale(mu, kb)
    o1, o2 = np.argsort(-lit, kind="stable"), np.argsort(-fold, kind="stable")
    diff = np.nonzero(o1 != o2)[0]
    # any reordering may only involve keys closer than the fold's rounding
    for i in diff:
        a, b = o1[i], o2[i]
        assert abs(lit[a] - lit[b]) < 1e-9 * max(scale[a], scale[b])
    assert np.array_equal(O.select_topb(lit, wl.budget), O.select_topb(fold, wl.budget))


def test_band_evaluation_count_factor():
    wl, inp, omega, qb, kb, delta = _c1_unit()
    D = O.power_of_two_offsets()
    c_lit, c_fold = {}, {}
    O.score_unfolded(qb, kb, delta, omega, D, counter=c_lit)
    W = O.fold_weights(omega, D, counter=c_fold)
    O.score_folded_complex(O.folded_center(qb, W), kb, delta, omega, counter=c_fold)
    n, f = kb.shape
    assert c_lit["band_cos"] == n * f * len(D)
    assert c_fold["band_cos"] == n * f and c_fold["weight_exp"] == f * len(D)
    assert c_lit["band_cos"] // c_fold["band_cos"] == 17


# --------------------------------------------------------------------------------------------
# Structure of the score (P3, P6)
# --------------------------------------------------------------------------------------------

def test_single_band_reduces_to_one_cosine_average():
    q, k, pos, t, omega = small_case(4, n=10, d=16)
    D = O.power_of_two_offsets()
    for f in [0, 3, 7]:
        qm, km = np.zeros_like(q), np.zeros_like(k)
        qm[2 * f:2 * f + 2], km[:, 2 * f:2 * f + 2] = q[2 * f:2 * f + 2], k[:, 2 * f:2 * f + 2]
        qb, kb = O.as_bands(qm), O.as_bands(km)
        mu = O.folded_center(qb, O.fold_weights(omega, D))
        got = O.score_folded_complex(mu, kb, t - pos, omega)
        for i in range(len(pos)):
            qa = math.hypot(q[2 * f], q[2 * f + 1])
            ka = math.hypot(k[i, 2 * f], k[i, 2 * f + 1])
            phi = math.atan2(q[2 * f + 1], q[2 * f]) - math.atan2(k[i, 2 * f + 1], k[i, 2 * f])
            ref = qa * ka * sum(math.cos(omega[f] * (t - pos[i] + dd) + phi) for dd in D) / len(D)
            assert abs(got[i] - ref) <= 1e-11 * qa * ka


def test_score_structure_invariants():
    q, k, pos, t, omega = small_case(5)
    D = O.power_of_two_offsets()
    W = O.fold_weights(omega, D)
    qb, kb = O.as_bands(q), O.as_bands(k)
    mu = O.folded_center(qb, W)
    s = O.score_folded_complex(mu, kb, t - pos, omega)
    sc = l1_scale(mu, kb)
    # linear in the center and in the key
    assert np.max(scaled_err(O.score_folded_complex(-3 * mu, kb, t - pos, omega), -3 * s, 3 * sc)) < 1e-13
    k2 = O.as_bands(np.random.default_rng(9).standard_normal(k.shape))
    s_sum = O.score_folded_complex(mu, kb + k2, t - pos, omega)
    s_2 = O.score_folded_complex(mu, k2, t - pos, omega)
    assert np.allclose(s_sum, s + s_2, atol=1e-12 * np.max(np.abs(s)))
    # a common rotation of center and key in each band changes nothing
    rot = np.exp(1j * np.random.default_rng(10).uniform(0, 2 * np.pi, size=qb.size))
    s_rot = O.score_folded_complex(O.folded_center(qb * rot, W), kb * rot[None, :], t - pos, omega)
    assert np.max(scaled_err(s_rot, s, sc)) < 1e-13
    # only the distance matters: shifting t and p together changes nothing
    s_shift = O.score_folded_complex(mu, kb, O.distances(t + 777, pos + 777), omega)
    assert np.array_equal(s_shift, s)
    # additive over bands
    parts = sum(O.score_folded_complex(mu[f:f + 1], kb[:, f:f + 1], t - pos, omega[f:f + 1])
                for f in range(qb.size))
    assert np.allclose(parts, s, atol=1e-12 * np.max(np.abs(s)))


def test_max_variant():
    q, k, pos, t, omega = small_case(6, n=12, d=8)
    D = O.power_of_two_offsets()
    qb, kb = O.as_bands(q), O.as_bands(k)
    delta = O.distances(t, pos)
    mx = O.score_unfolded_max(qb, kb, delta, omega, D)
    mean = O.score_unfolded(qb, kb, delta, omega, D)
    assert np.all(mx >= mean - 1e-12)
    # one offset: the max is the score at that offset
    assert np.allclose(O.score_unfolded_max(qb, kb, delta, omega, [4]),
                       O.score_unfolded(qb, kb, delta, omega, [4]), atol=1e-12)
    # against rotation matrices: max over offsets of the future rotary logit
    kr = rope_rotate(k, pos, omega)
    per = []
    for off in D:
        qr = rope_rotate(np.repeat(q[None, :], len(pos), 0), np.full(len(pos), t + off), omega)
        per.append(np.sum(qr * kr, axis=1))
    assert np.allclose(mx, np.max(per, axis=0), atol=1e-11 * np.max(np.abs(per)))


def test_post_rope_form():
    q, k, pos, t, omega = small_case(7)
    D = O.power_of_two_offsets()
    mu = O.folded_center(O.as_bands(q), O.fold_weights(omega, D))
    direct = O.score_folded_complex(mu, O.as_bands(k), t - pos, omega)
    rotated = O.as_bands(rope_rotate(k, pos, omega))  # keys as a rotary cache stores them
    assert np.allclose(O.rotate_keys(O.as_bands(k), pos, omega), rotated, atol=1e-12)
    got = O.score_post_rope(mu, rotated, t, omega)
    assert np.max(scaled_err(got, direct, l1_scale(mu, O.as_bands(k)))) < 1e-11


# --------------------------------------------------------------------------------------------
# Select (P7, P8) and compaction (P9)
# --------------------------------------------------------------------------------------------

def _dominates(si, sj, i, j):
    """Row i outranks row j: NaN is below everything; -0 == +0; ties go to the lower index."""
    ni, nj = math.isnan(si), math.isnan(sj)
    if ni != nj:
        return nj
    if ni and nj:
        return i < j
    if si != sj:
        return si > sj
    return i < j


@pytest.mark.parametrize("seed", range(40))
def test_select_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(0, 11))
    pool = np.array([0.0, -0.0, 1.5, -1.5, 2.0, np.nan, -np.inf, np.inf, 0.25])
    s = np.where(rng.random(n) < 0.5, rng.choice(pool, size=n), rng.standard_normal(n))
    for B in [0, 1, 3, n, n + 2]:
        m = min(B, n)
        valid = [set(c) for c in itertools.combinations(range(n), m)
                 if all(_dominates(s[i], s[j], i, j) for i in c for j in range(n) if j not in c)]
        assert len(valid) == 1
        got = O.select_topb(s, B)
        assert set(got.tolist()) == valid[0]
        assert np.all(np.diff(got) > 0)


def test_select_zero_center_keeps_first_rows():
    q, k, pos, t, omega = small_case(8, n=40)
    mu = np.zeros(q.size // 2, dtype=np.complex128)
    s = O.score_folded_complex(mu, O.as_bands(k), t - pos, omega)
    assert np.all(s == 0)
    s[::3] = -0.0
    assert O.select_topb(s, 7).tolist() == list(range(7))


def test_select_matches_full_sort():
    s = np.random.default_rng(11).standard_normal(5000)
    s[::7] = s[3]  # heavy ties
    kept = O.select_topb(s, 600)
    order = sorted(range(s.size), key=lambda i: (-s[i], i))
    assert kept.tolist() == sorted(order[:600])


def test_compaction_is_a_gather():
    rng = np.random.default_rng(12)
    rows = f32_to_bf16_bits(rng.standard_normal((50, 8)).astype(np.float32))
    kept = np.array([1, 4, 5, 30, 49])
    out = O.compact_rows(rows, kept, 8, np.uint16(0))
    assert np.array_equal(out[:5], np.take(rows, kept, axis=0))
    assert np.all(out[5:] == 0)
    assert out.dtype == rows.dtype


def test_unit_pass_end_to_end_small():
    wl = workload("c2")
    packed = pack_units(wl, units=[3], lengths=[600])
    res = O.unit_pass(packed["centers"][0], packed["keys"], packed["values"], packed["pos"],
                      int(packed["t"][0]), wl.d, wl.theta, O.power_of_two_offsets(), 64)
    kept = res["kept"]
    assert kept.size == 64 and np.all(np.diff(kept) > 0)
    assert np.array_equal(res["K_out"], packed["keys"][kept])
    assert np.array_equal(res["pos_out"], kept.astype(np.int32))
    s = res["scores"]
    assert np.min(s[kept]) >= np.max(np.delete(s, kept))
