"""GPU parity of the in-place pass (tri_prune_inplace): one pass over fresh units, and the steady
state of chat serving, where each 1024-row prefill chunk appended to B kept rows is pruned back
to B with sparse positions.

Expected result of a pass, from the GPU's own scores (the select is exact on them) and the
arrangement rule of the header: kept rows below m stay; the freed slots below m, lowest first,
receive the kept rows at or beyond m, highest first. Scores are checked against the fp64 oracle
(scaled error <= 2e-3) and the kept set against the oracle's outside the tolerance band.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from synthgen import unit_inputs, workload
from tests._parity import SPLIT_ROWS, TOL, keys_to_device, keys_to_host, kept_mismatch, score_error, widen

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def arrangement(kept, m):
    """Source row of each of the first m slots after the moves."""
    kept = np.asarray(kept, dtype=np.int64)
    stay = kept[kept < m]
    movers = np.sort(kept[kept >= m])[::-1]
    free = np.setdiff1d(np.arange(m), stay)
    assert free.size == movers.size
    src = np.arange(m)
    src[free] = movers
    return src


def oracle_scores(keys_bits, pos, t, center, wl):
    omega = O.rotary_frequencies(wl.d, wl.theta)
    kb = O.as_bands(widen(keys_bits, wl.dtype))
    mu = O.folded_center(O.as_bands(np.asarray(center, dtype=np.float32).astype(np.float64)),
                         O.fold_weights(omega, O.power_of_two_offsets()))
    s = O.score_folded_complex(mu, kb, O.distances(int(t), pos), omega)
    scale = np.sum(np.abs(mu)[None, :] * np.abs(kb), axis=1) / kb.shape[1]
    return s, scale


class Cache:
    """Host copy of a packed cache and the same cache on the device."""

    def __init__(self, wl, K, V, pos, lengths, t, centers):
        import rotary_frequency_key_amd as tri

        self.wl, self.dev = wl, torch.device("cuda:0")
        self.K, self.V, self.pos = K.copy(), V.copy(), pos.copy()
        self.lengths = np.asarray(lengths, dtype=np.int64)
        self.row_off = np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int64)
        self.t = np.asarray(t, dtype=np.int32)
        self.centers = centers
        _, mu = tri.tri_fold_weights(wl.d, wl.theta, O.power_of_two_offsets(), centers)
        self.mu = mu

    def run(self, B, max_rows=None):
        import rotary_frequency_key_amd as tri

        d = self.dev
        K = keys_to_device(self.K, self.wl.dtype, d)
        V = keys_to_device(self.V, self.wl.dtype, d)
        pos = torch.from_numpy(self.pos).to(d)
        if max_rows is None:
            max_rows = int(self.lengths.max()) if self.lengths.size else 0
        scores, kept_cnt = tri.prune_inplace(K, V, pos, torch.from_numpy(self.row_off).to(d), max_rows,
                                             torch.from_numpy(self.t).to(d), torch.from_numpy(self.mu).to(d),
                                             self.wl.theta, B)
        torch.cuda.synchronize()
        return (scores.cpu().numpy(), kept_cnt.cpu().numpy(), keys_to_host(K, self.wl.dtype),
                keys_to_host(V, self.wl.dtype), pos.cpu().numpy())

    def check_pass(self, B, label, max_rows=None):
        """Run one in-place pass and check it; then adopt the expected arrangement."""
        scores, kept_cnt, K, V, pos = self.run(B, max_rows)
        worst, self.mism, self.moved = 0.0, 0, 0
        self.scores = scores
        for u in range(len(self.lengths)):
            a, b = self.row_off[u], self.row_off[u + 1]
            n = b - a
            m = min(B, n)
            assert kept_cnt[u] == m, (label, u)
            s_ref, scale = oracle_scores(self.K[a:b], self.pos[a:b], self.t[u], self.centers[u], self.wl)
            err = score_error(scores[a:b], s_ref, scale)
            worst = max(worst, err)
            assert err <= TOL, (label, u, err)
            kept = O.select_topb(scores[a:b], B)  # exact on the GPU's own scores
            self.mism += kept_mismatch(kept, s_ref, scale, B)
            src = arrangement(kept, m)
            assert np.array_equal(K[a:a + m], self.K[a:b][src]), (label, u)
            assert np.array_equal(V[a:a + m], self.V[a:b][src]), (label, u)
            assert np.array_equal(pos[a:a + m], self.pos[a:b][src]), (label, u)
            # rows from m on are left as they were
            assert np.array_equal(K[a + m:b], self.K[a + m:b]), (label, u)
            assert np.array_equal(pos[a + m:b], self.pos[a + m:b]), (label, u)
            moved = int(np.sum(src != np.arange(m)))
            assert moved <= min(m, n - m)
            self.moved += moved
        self.K, self.V, self.pos = K, V, pos
        return worst


@pytest.mark.parametrize("max_rows", [None, SPLIT_ROWS])
def test_inplace_single_pass_edges(max_rows):
    """Ragged units in one call: empty, shorter than B, equal to B, and longer; budgets 0, 1 and
    more."""
    wl = dataclasses.replace(workload("c2"), heads=6)
    lengths = [0, 7, 300, 1000, 4100, 20000]
    parts = [unit_inputs(wl, u, n) for u, n in enumerate(lengths)]
    K = np.concatenate([p["keys"] for p in parts])
    V = np.concatenate([p["values"] for p in parts])
    pos = np.concatenate([p["pos"] for p in parts]).astype(np.int32)
    centers = np.stack([p["center"] for p in parts])
    for B in [0, 1, 300, 2500]:
        say(f"case in-place single pass B={B} max_rows={max_rows}")
        c = Cache(wl, K, V, pos, lengths, [max(n, 1) for n in lengths], centers)
        c.check_pass(B, f"single B={B}", max_rows)


@pytest.mark.parametrize("dtype,max_rows", [("bf16", None), ("f32", None), ("bf16", SPLIT_ROWS)])
def test_inplace_steady_state(dtype, max_rows):
    """Pass 0 prunes 20000 rows per unit to B = 3000; then three times a 1024-row chunk with the
    next positions is appended and the 4024 rows are pruned back to 3000."""
    wl = dataclasses.replace(workload("c5"), dtype=dtype, seqs=1, layers=1, heads=4)
    U, N0, B, chunk, passes = 4, 20000, 3000, 1024, 3
    total = N0 + passes * chunk
    parts = [unit_inputs(wl, u, total) for u in range(U)]
    centers = np.stack([p["center"] for p in parts])
    say(f"case in-place steady state {dtype}: pass 0")
    K = np.concatenate([p["keys"][:N0] for p in parts])
    V = np.concatenate([p["values"][:N0] for p in parts])
    pos = np.concatenate([p["pos"][:N0] for p in parts]).astype(np.int32)
    c = Cache(wl, K, V, pos, [N0] * U, [N0] * U, centers)
    c.check_pass(B, "pass 0", max_rows)
    for k in range(1, passes + 1):
        lo, hi = N0 + (k - 1) * chunk, N0 + k * chunk
        Kn, Vn, Pn = [], [], []
        for u in range(U):
            a = c.row_off[u]
            Kn += [c.K[a:a + B], parts[u]["keys"][lo:hi]]
            Vn += [c.V[a:a + B], parts[u]["values"][lo:hi]]
            Pn += [c.pos[a:a + B], parts[u]["pos"][lo:hi].astype(np.int32)]
        t = hi
        c = Cache(wl, np.concatenate(Kn), np.concatenate(Vn), np.concatenate(Pn), [B + chunk] * U, [t] * U, centers)
        say(f"case in-place steady state {dtype}: pass {k} (positions sparse: {np.unique(np.diff(np.sort(c.pos[:B]))).size} gaps)")
        err = c.check_pass(B, f"pass {k}", max_rows)
        say(f"   worst score error {err:.3g}, {c.moved} rows moved")
        # the bench's count of moved rows, from the scores alone, agrees with the moves made
        import bench
        sc = torch.from_numpy(c.scores.reshape(U, B + chunk).copy())
        assert int(bench.count_moved_rows(torch, sc, B).item()) == c.moved, (k, c.moved)
        say(f"[margin] in-place steady state ({dtype}, 4 units, {B} + {chunk} rows, pass {k}"
            f"{', max_rows ' + str(max_rows) if max_rows else ''}) | {err:.3g} | {c.mism} | {U}")


def test_inplace_rotated_keys_without_positions():
    """Rotated keys with no position array: the same rows move as with positions."""
    import rotary_frequency_key_amd as tri

    wl = dataclasses.replace(workload("c2"), heads=2)
    parts = [unit_inputs(wl, u, 5000) for u in range(2)]
    K = np.concatenate([p["keys"] for p in parts])
    V = np.concatenate([p["values"] for p in parts])
    centers = np.stack([p["center"] for p in parts])
    dev = torch.device("cuda:0")
    _, mu = tri.tri_fold_weights(wl.d, wl.theta, O.power_of_two_offsets(), centers)
    row_off = torch.tensor([0, 5000, 10000], dtype=torch.int64, device=dev)
    t = torch.tensor([5000, 5000], dtype=torch.int32, device=dev)
    out = []
    for with_pos in [True, False]:
        Kd, Vd = keys_to_device(K, "bf16", dev), keys_to_device(V, "bf16", dev)
        pos = torch.from_numpy(np.concatenate([p["pos"] for p in parts]).astype(np.int32)).to(dev) if with_pos else None
        scores, cnt = tri.prune_inplace(Kd, Vd, pos, row_off, 5000, t, torch.from_numpy(mu).to(dev), wl.theta, 700,
                                        layout=tri.TRI_KEYS_ROTATED)
        torch.cuda.synchronize()
        out.append((scores.cpu().numpy(), keys_to_host(Kd, "bf16"), keys_to_host(Vd, "bf16")))
    assert np.array_equal(out[0][0], out[1][0])
    assert np.array_equal(out[0][1], out[1][1]) and np.array_equal(out[0][2], out[1][2])
    for u in range(2):
        kept = O.select_topb(out[0][0][u * 5000:(u + 1) * 5000], 700)
        src = arrangement(kept, 700)
        assert np.array_equal(out[0][1][u * 5000:u * 5000 + 700], K[u * 5000:(u + 1) * 5000][src])
