"""Shared helpers of the GPU parity tests: move generated inputs to the device, run the pass
through the C interface, and compute the fp64 oracle's reference for a unit.

Score tolerance: scaled error e_k = |s_gpu - s_ref| / max(|s_ref|, L1_k / F) <= 2e-3, with
L1_k = sum_f |mu'_f| |k_f|. The plain relative error is meaningless for scores whose band
terms cancel to near zero; L1_k / F is the magnitude of one band's term.
"""
import os

import numpy as np
import torch

import oracle as O

TOL = 2e-3

# The library picks its select kernels from max_rows: units of up to 2^18 rows take the fused
# resolve-and-emit kernel (the in-place pass, up to 2^16 rows: one workgroup per unit with the
# keys in registers); longer units take the candidate / resolve / emit (or mark) kernels. max_rows
# is only an upper bound on the unit lengths, so passing this value runs the second path on
# short units.
SPLIT_ROWS = (1 << 18) + 1


def gen_workers():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(16, n or 1))


def keys_to_device(arr, dtype, dev):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(dev)


def keys_to_host(t, dtype):
    if dtype == "bf16":
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy()


def run_gpu(P, wl, B, *, layout=0, centers=None, theta=None, offsets=None,
            keys=None, max_rows=None, path="fused"):
    """One pass through the library. Returns a dict of host numpy arrays."""
    import rotary_frequency_key_amd as tri

    dev = torch.device("cuda:0")
    theta = wl.theta if theta is None else theta
    offsets = O.power_of_two_offsets() if offsets is None else offsets
    centers = P["centers"] if centers is None else centers
    _, mu = tri.tri_fold_weights(wl.d, theta, offsets, centers)
    K = keys_to_device(P["keys"] if keys is None else keys, wl.dtype, dev)
    V = keys_to_device(P["values"], wl.dtype, dev)
    pos = torch.from_numpy(P["pos"]).to(dev)
    row_off = torch.from_numpy(P["row_off"]).to(dev)
    t_now = torch.from_numpy(P["t"]).to(dev)
    mu_d = torch.from_numpy(mu).to(dev)
    U = len(P["row_off"]) - 1
    lens = np.diff(P["row_off"])
    if max_rows is None:
        max_rows = int(lens.max()) if lens.size else 0
    ws = tri.make_workspace(U, max_rows, dev) if path != "noalloc" else None
    # sentinel-filled outputs: rows past kept_cnt must stay untouched
    K_out = torch.full((U, B, wl.d), 123.5, dtype=K.dtype, device=dev)
    V_out = torch.full_like(K_out, -77.0)
    pos_out = torch.full((U, B), -5, dtype=torch.int32, device=dev)
    if path == "fused":  # tri_prune_pass
        scores, kept_idx, kept_cnt, K_out, V_out, pos_out = tri.prune_pass(
            K, V, pos, row_off, max_rows, t_now, mu_d, theta, B, ws=ws, K_out=K_out, V_out=V_out,
            pos_out=pos_out, layout=layout)
    elif path == "noalloc":  # tri_prune_pass_noalloc: the library's static workspace, not ws
        scores, kept_idx, kept_cnt, K_out, V_out, pos_out = tri.prune_pass_noalloc(
            K, V, pos, row_off, max_rows, t_now, mu_d, theta, B, K_out=K_out, V_out=V_out,
            pos_out=pos_out, layout=layout)
    elif path == "calls":  # tri_score (histogram) -> tri_select_topb -> tri_compact_kv
        scores, kept_idx, kept_cnt, K_out, V_out, pos_out = tri.prune_pass_3calls(
            K, V, pos, row_off, max_rows, t_now, mu_d, theta, B, ws=ws, K_out=K_out, V_out=V_out,
            pos_out=pos_out, layout=layout)
    else:  # tri_score without histogram -> standalone tri_select_topb -> tri_compact_kv
        scores = tri.tri_score(K, row_off, max_rows, pos, t_now, mu_d, theta, layout=layout)
        kept_idx, kept_cnt = tri.tri_select_topb(scores, row_off, max_rows, B, ws=ws)
        K_out, V_out, pos_out = tri.tri_compact_kv(K, V, pos, row_off, kept_idx, kept_cnt, B,
                                                   K_out=K_out, V_out=V_out, pos_out=pos_out)
    torch.cuda.synchronize()
    out = {
        "scores": scores.cpu().numpy(),
        "kept_idx": kept_idx.cpu().numpy(),
        "kept_cnt": kept_cnt.cpu().numpy(),
        "K_out": keys_to_host(K_out, wl.dtype),
        "V_out": keys_to_host(V_out, wl.dtype),
        "pos_out": pos_out.cpu().numpy(),
        "mu": mu,
    }
    out["ws_after"] = ws_at_rest(ws.cpu().numpy(), U) if ws is not None else None
    return out


def ws_at_rest(ws, U):
    """True when the workspace is in its rest state: the per-unit top-digit histograms (its
    first U * 4096 words) are zero. The rest of the workspace is scratch."""
    return bool(np.all(ws.view(np.uint32)[:U * 4096] == 0))


def widen(keys, dtype):
    return O.widen_bf16(keys) if dtype == "bf16" else np.asarray(keys, dtype=np.float32).astype(np.float64)


def order_keys(scores):
    """Monotone u32 keys of binary32 scores (-0 == +0, NaN lowest), as the select compares them."""
    b = np.asarray(scores, dtype=np.float32).view(np.uint32).astype(np.uint64)
    mag = b & 0x7FFFFFFF
    k = np.where(b & 0x80000000, (~b) & 0xFFFFFFFF, b | 0x80000000)
    k = np.where(mag == 0, 0x80000000, k)
    k = np.where(mag > 0x7F800000, 0, k)
    return k.astype(np.uint64)


def candidate_profile(scores, B, rows_per_group=1024):
    """Select-path facts for one unit's scores: the number of keys sharing the B-th key's top 12
    bits (candidates), the largest number of them in one group of rows, and the number sharing
    its top 22 bits. Used to show that a test reaches the code path it is meant for."""
    k = order_keys(scores)
    m = min(B, k.size)
    T = np.sort(k)[::-1][m - 1]
    cand = (k >> 20) == (T >> 20)
    per = np.add.reduceat(cand.astype(np.int64), np.arange(0, k.size, rows_per_group))
    return int(cand.sum()), int(per.max()), int(np.sum((k >> 10) == (T >> 10)))


def oracle_unit(P, i, wl, theta=None, offsets=None, centers=None, layout="interleaved"):
    """fp64 reference scores of unit i and the per-key tolerance scale L1_k / F."""
    theta = wl.theta if theta is None else theta
    offsets = O.power_of_two_offsets() if offsets is None else offsets
    centers = P["centers"] if centers is None else centers
    a, b = P["row_off"][i], P["row_off"][i + 1]
    omega = O.rotary_frequencies(wl.d, theta)
    qb = O.as_bands(np.asarray(centers[i], dtype=np.float32).astype(np.float64), layout)
    kb = O.as_bands(widen(P["keys"][a:b], wl.dtype), layout)
    mu = O.folded_center(qb, O.fold_weights(omega, offsets))
    s = O.score_folded_complex(mu, kb, O.distances(int(P["t"][i]), P["pos"][a:b]), omega)
    scale = np.sum(np.abs(mu)[None, :] * np.abs(kb), axis=1) / max(kb.shape[1], 1)
    return s, scale


def score_error(s_gpu, s_ref, scale):
    if s_ref.size == 0:
        return 0.0
    return float(np.max(np.abs(s_gpu.astype(np.float64) - s_ref) / np.maximum(np.abs(s_ref), scale)))


def kept_mismatch(kept_gpu, s_ref, scale, B):
    """Keys on which the GPU's kept set and the oracle's differ. Every such key must lie within
    the tolerance band around the oracle's B-th score. Returns the number of such keys."""
    kept_ref = O.select_topb(s_ref, B)
    diff = sorted(set(kept_gpu.tolist()) ^ set(kept_ref.tolist()))
    if diff:
        star = kept_ref[np.argmin(s_ref[kept_ref])]
        for k in diff:
            band = TOL * max(scale[k], scale[star])
            assert abs(s_ref[k] - s_ref[star]) <= band, (k, s_ref[k], s_ref[star], band)
    return len(diff)


def check_unit(P, i, wl, out, B, s_ref=None, scale=None, label=""):
    """All per-unit checks; returns (score error, kept mismatches)."""
    a, b = P["row_off"][i], P["row_off"][i + 1]
    n = b - a
    m = min(B, n)
    s_gpu = out["scores"][a:b]
    if s_ref is None:
        s_ref, scale = oracle_unit(P, i, wl)
    err = score_error(s_gpu, s_ref, scale)
    assert err <= TOL, f"{label} unit {i}: score error {err:.3g}"
    assert out["kept_cnt"][i] == m, label
    kept = out["kept_idx"][i, :m]
    # select is exact on the GPU's own scores
    assert np.array_equal(kept, O.select_topb(s_gpu, B)), f"{label} unit {i}: select != top-B of own scores"
    assert np.all(out["kept_idx"][i, m:] == -1), label
    mism = kept_mismatch(kept, s_ref, scale, B)
    # compaction is a byte copy of the kept rows; rows past the count are untouched
    assert np.array_equal(out["K_out"][i, :m], P["keys"][a:b][kept]), label
    assert np.array_equal(out["V_out"][i, :m], P["values"][a:b][kept]), label
    assert np.array_equal(out["pos_out"][i, :m], P["pos"][a:b][kept]), label
    assert np.all(out["pos_out"][i, m:] == -5), label
    assert np.all(widen(out["K_out"][i, m:], wl.dtype) == 123.5), label
    assert np.all(widen(out["V_out"][i, m:], wl.dtype) == -77.0), label
    return err, mism
