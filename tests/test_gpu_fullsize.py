"""The two largest workloads at full size, generated on the device (synthgen.device):
4096 ragged units of 8192..65536 keys (B = 2048) and 2048 units of 132096 keys (B = 12000).

Every unit is checked on the device for properties that hold at any size (kept counts; kept
indices ascending, in range and padded with -1; no dropped key above a kept one, and among equal
scores the kept ones below the dropped ones; compaction a byte copy); a sample of units is
copied back and checked against the fp64 oracle (scores within the tolerance, the kept set
outside the tolerance band).
"""
import numpy as np
import pytest
import torch

import oracle as O
from synthgen import workload
from synthgen.device import device_workload
from tests._parity import TOL, kept_mismatch, score_error, widen

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def unit_properties(scores, row_off_d, lengths, kept_idx, kept_cnt, B, dev):
    """Device-side checks of every unit's select result against its own scores."""
    U = lengths.size
    n = torch.from_numpy(lengths).to(dev)
    m = torch.clamp(n, max=B)
    assert torch.equal(kept_cnt.to(torch.int64), m)
    j = torch.arange(B, device=dev)[None, :]
    valid = j < m[:, None]
    assert torch.all(kept_idx[~valid] == -1)
    ki = kept_idx.to(torch.int64)
    assert bool(torch.all(((ki >= 0) & (ki < n[:, None])) | ~valid))
    # ascending within each unit
    assert bool(torch.all((ki[:, 1:] > ki[:, :-1]) | ~valid[:, 1:]))
    # kept mask over all rows
    R = scores.numel()
    starts = row_off_d[:-1]
    rows = (starts[:, None] + ki)[valid]
    kept = torch.zeros(R, dtype=torch.bool, device=dev)
    kept[rows] = True
    unit = torch.repeat_interleave(torch.arange(U, device=dev), n)
    s = scores.to(torch.float64)
    inf = torch.full((U,), float("inf"), dtype=torch.float64, device=dev)
    min_kept = inf.clone().scatter_reduce(0, unit[kept], s[kept], reduce="amin")
    max_drop = (-inf).clone().scatter_reduce(0, unit[~kept], s[~kept], reduce="amax")
    assert torch.all(min_kept >= max_drop), "a dropped key scores above a kept one"
    # equal scores at the threshold: kept rows below dropped rows
    tie = (min_kept == max_drop)
    if torch.any(tie):
        local = torch.arange(R, device=dev) - starts[unit]
        at_t = s == min_kept[unit]
        big = torch.full((U,), R, dtype=torch.int64, device=dev)
        last_kept = torch.full((U,), -1, dtype=torch.int64, device=dev).scatter_reduce(
            0, unit[kept & at_t], local[kept & at_t], reduce="amax")
        first_drop = big.scatter_reduce(0, unit[~kept & at_t], local[~kept & at_t], reduce="amin")
        assert torch.all(~tie | (last_kept < first_drop)), "ties not kept lowest rows first"
    return kept


def check_sample(W, wl, out_scores, kept_idx, B, u):
    a, b = int(W["row_off"][u]), int(W["row_off"][u + 1])
    keys = W["K"][a:b]
    keys_h = keys.cpu().view(torch.int16).numpy().view(np.uint16) if wl.dtype == "bf16" else keys.cpu().numpy()
    pos = W["pos"][a:b].cpu().numpy()
    omega = O.rotary_frequencies(wl.d, wl.theta)
    kb = O.as_bands(widen(keys_h, wl.dtype))
    mu = O.folded_center(O.as_bands(W["centers"][u].astype(np.float64)), O.fold_weights(omega, O.power_of_two_offsets()))
    s_ref = O.score_folded_complex(mu, kb, O.distances(int(W["t"][u]), pos), omega)
    scale = np.sum(np.abs(mu)[None, :] * np.abs(kb), axis=1) / kb.shape[1]
    s_gpu = out_scores[a:b].cpu().numpy()
    err = score_error(s_gpu, s_ref, scale)
    assert err <= TOL, (u, err)
    m = min(B, b - a)
    kept = kept_idx[u, :m].cpu().numpy()
    assert np.array_equal(kept, O.select_topb(s_gpu, B))
    mism = kept_mismatch(kept, s_ref, scale, B)
    return err, mism


@pytest.mark.parametrize("name", ["c4", "c5"])
def test_full_size_sampled(name):
    import rotary_frequency_key_amd as tri

    dev = torch.device("cuda:0")
    wl = workload(name)
    say(f"case {name} full size: generating {wl.n_units} units on the device")
    W = device_workload(wl, dev)
    U, B = wl.n_units, wl.budget
    lengths = W["lengths"]
    max_rows = int(lengths.max())
    say(f"   {int(W['row_off'][-1])} keys, max {max_rows} per unit; running the pass")
    _, mu = tri.tri_fold_weights(wl.d, wl.theta, O.power_of_two_offsets(), W["centers"])
    ws = tri.make_workspace(U, max_rows, dev)
    scores, kept_idx, kept_cnt, K_out, V_out, pos_out = tri.prune_pass(
        W["K"], W["V"], W["pos"], W["row_off_d"], max_rows, W["t_d"], torch.from_numpy(mu).to(dev), wl.theta, B,
        ws=ws)
    torch.cuda.synchronize()
    assert bool(torch.all(ws[:U * 4096 * 4] == 0)), "workspace back at rest"
    say("   every unit: counts, order, threshold, ties")
    unit_properties(scores, W["row_off_d"], lengths, kept_idx, kept_cnt, B, dev)
    say("   every unit: compaction")
    m = torch.clamp(torch.from_numpy(lengths).to(dev), max=B)
    valid = torch.arange(B, device=dev)[None, :] < m[:, None]
    src = (W["row_off_d"][:-1][:, None] + kept_idx.to(torch.int64).clamp(min=0))
    bits = torch.int16 if wl.dtype == "bf16" else torch.int32  # compare bit patterns
    for u0 in range(0, U, 256):  # in slices, to bound the temporaries
        sl = slice(u0, min(U, u0 + 256))
        v = valid[sl]
        assert torch.equal(K_out[sl][v].view(bits), W["K"][src[sl][v]].view(bits))
        assert torch.equal(V_out[sl][v].view(bits), W["V"][src[sl][v]].view(bits))
        assert torch.equal(pos_out[sl][v], W["pos"][src[sl][v]])
    rng = np.random.default_rng(7)
    sample = sorted(set([0, U // 2, U - 1] + rng.choice(U, size=3, replace=False).tolist()))
    worst, total = 0.0, 0
    for u in sample:
        err, mism = check_sample(W, wl, scores, kept_idx, B, u)
        worst, total = max(worst, err), total + mism
        say(f"   unit {u} (N={lengths[u]}): score error {err:.3g}, kept mismatches {mism}")
    say(f"[margin] {name.upper()} sample ({U} units, {int(lengths.min())}..{max_rows} keys, B={B}) | {worst:.3g} | "
        f"{total} | {len(sample)}")
